// mk_device.h — device helpers shared by the HIP kernels of libmk (gfx950 only).
//
// Packed Q4_K-style layout (library-defined; 144 B per 256 weights as in the
// block format of the workload definition, rows padded to 64):
//   matrix = 64-row tiles, each tile = n_in/256 "units" in superblock order;
//   unit (tile, b) = 9216 B:
//     [0, 1024)                  header block: row r (0..63) at r*16:
//                                  u16 d, u16 dmin (fp16 bits),
//                                  bytes 4..11: byte 4+j = sc_j | (m_j >> 4) << 6
//                                  bytes 12..15: byte 12+i = (m_i & 15) | (m_{i+4} & 15) << 4
//     [1024 + j*1024, +1024)     codes of sub-block j: row r at r*16, 16 B:
//                                  dword w, byte i: low nibble = code 8w+i,
//                                                   high nibble = code 8w+4+i
// so that (w & 0x0F0F0F0F) and ((w >> 4) & 0x0F0F0F0F) are the int8 operands
// for codes 8w..8w+3 and 8w+4..8w+7, in the same order as the activations.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

constexpr int kTileRows = 64;
constexpr int kUnitBytes = 9216;
constexpr int kHdrBytes = 1024;
constexpr int kSubBytes = 1024;

typedef const uint32_t __attribute__((address_space(4))) cu32;
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef const u32x8 __attribute__((address_space(4))) cu32x8;
typedef const float __attribute__((address_space(4))) cf32;
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef const f32x8 __attribute__((address_space(4))) cf32x8;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Reads through the scalar cache: only for data that no wave of the running
// kernel writes before the read (the caller guarantees this).
template <typename T>
__device__ __forceinline__ const T __attribute__((address_space(4)))* as_const(const void* p) {
  return (const T __attribute__((address_space(4)))*)(uintptr_t)p;
}

// Wave-uniform copies (the value is the same in every lane; this tells the
// compiler so, which keeps it in scalar registers).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ T* uniform(T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Data shared between workgroups of one launch is stored and loaded with
// device-scope (sc1) accesses, which are coherent across the XCDs' L2
// caches without whole-cache write-back or invalidation.
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_i8(int8_t* p, int8_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_coh_i(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The atomic may only be performed once this wave's stores are in memory.  A
// workgroup-scope release fence does not wait for them on this target (the
// waves of a workgroup share one L1), so the wait is explicit; with every
// shared store device-scope (sc1), completion means visibility to all CUs.
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ unsigned ticket_add(unsigned* p, unsigned n = 1u) {
  stores_done();
  return __hip_atomic_fetch_add(p, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Decoded header of one (row, superblock): dsc[j] = d*sc_j, dm[j] = dmin*m_j.
struct Hdr {
  float dsc[8];
  float dm[8];
};

__device__ __forceinline__ void decode_hdr(const u32x4 h, Hdr& o) {
  const float d = f16_bits_to_f32(h.x & 0xffffu);
  const float dmin = f16_bits_to_f32(h.x >> 16);
  const uint32_t sc03 = h.y & 0x3F3F3F3Fu, sc47 = h.z & 0x3F3F3F3Fu;
  const uint32_t m03 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
  const uint32_t m47 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o.dsc[j] = d * (float)((sc03 >> (8 * j)) & 0xffu);
    o.dsc[j + 4] = d * (float)((sc47 >> (8 * j)) & 0xffu);
    o.dm[j] = dmin * (float)((m03 >> (8 * j)) & 0xffu);
    o.dm[j + 4] = dmin * (float)((m47 >> (8 * j)) & 0xffu);
  }
}

// 16-B streaming load (nontemporal: the weight stream is read once).
__device__ __forceinline__ u32x4 ldg16_nt(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

// Integer dot product of one sub-block row (32 codes, 16 B) with 32 int8
// activations (8 dwords in natural order).  Exact.
__device__ __forceinline__ int dot_sub(const u32x4 c, const u32x8 a) {
  int p = 0;
  p = __builtin_amdgcn_sdot4((int)(c.x & 0x0F0F0F0Fu), (int)a[0], p, false);
  p = __builtin_amdgcn_sdot4((int)((c.x >> 4) & 0x0F0F0F0Fu), (int)a[1], p, false);
  p = __builtin_amdgcn_sdot4((int)(c.y & 0x0F0F0F0Fu), (int)a[2], p, false);
  p = __builtin_amdgcn_sdot4((int)((c.y >> 4) & 0x0F0F0F0Fu), (int)a[3], p, false);
  p = __builtin_amdgcn_sdot4((int)(c.z & 0x0F0F0F0Fu), (int)a[4], p, false);
  p = __builtin_amdgcn_sdot4((int)((c.z >> 4) & 0x0F0F0F0Fu), (int)a[5], p, false);
  p = __builtin_amdgcn_sdot4((int)(c.w & 0x0F0F0F0Fu), (int)a[6], p, false);
  p = __builtin_amdgcn_sdot4((int)((c.w >> 4) & 0x0F0F0F0Fu), (int)a[7], p, false);
  return p;
}

// Quantized activation rows as the GEMV engines consume them:
//   a8  [T][K] int8
//   ssg [K/32][16] float2 = (s, s * gsum) of group g for rows t = 0..15
//       (rows t >= T hold zeros, so padded matrix-core columns add nothing).
constexpr int kTPad = 16;
struct QAct {
  const int8_t* a8;
  const float* ssg;  // interleaved (s, s*gsum) pairs, [K/32][16][2]
  int32_t K;
  int32_t T;
};

// One 64-row unit (tile, superblock) of codes and its header, in registers.
struct Unit {
  u32x4 h;
  u32x4 c[8];
};

__device__ __forceinline__ void load_unit(const uint8_t* __restrict__ u, int lane, Unit& x) {
  x.h = ldg16_nt(u + lane * 16);
#pragma unroll
  for (int j = 0; j < 8; ++j) x.c[j] = ldg16_nt(u + kHdrBytes + j * kSubBytes + lane * 16);
}

// dot4 engine on one unit: lane = output row of the tile; the T activation
// rows are wave-uniform and read through the scalar cache.  Per (t, j):
//   acc[t] += s[t][g] * (d*sc_j) * P  -  (dmin*m_j) * (s*gsum)[t][g]
// with P the exact integer sub-block sum.
template <int T>
__device__ __forceinline__ void dot4_unit(const Unit& x, int b, const QAct& act, float (&acc)[T]) {
  Hdr hd;
  decode_hdr(x.h, hd);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int g = b * 8 + j;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const u32x8 a = *as_const<u32x8>(act.a8 + (size_t)t * act.K + (size_t)g * 32);
      const f32x2 ss = *as_const<f32x2>(act.ssg + ((size_t)g * kTPad + t) * 2);
      const int p = dot_sub(x.c[j], a);
      acc[t] = __builtin_fmaf((float)p * hd.dsc[j], ss.x, acc[t]);
      acc[t] = __builtin_fmaf(-hd.dm[j], ss.y, acc[t]);
    }
  }
}

// Accumulates units [b0, b1) of one tile with the next unit's loads issued
// before the current unit's arithmetic.  u0 already holds unit b0.
template <int T>
__device__ __forceinline__ void dot4_range_from(const uint8_t* __restrict__ tile, int b0, int b1, const QAct& act,
                                                int lane, float (&acc)[T], Unit& u0) {
  Unit u1;  // ping-pong buffers: no register copies between iterations
  for (int b = b0; b < b1; b += 2) {
    if (b + 1 < b1) load_unit(tile + (size_t)(b + 1) * kUnitBytes, lane, u1);
    dot4_unit<T>(u0, b, act, acc);
    if (b + 1 >= b1) break;
    if (b + 2 < b1) load_unit(tile + (size_t)(b + 2) * kUnitBytes, lane, u0);
    dot4_unit<T>(u1, b + 1, act, acc);
  }
}

template <int T>
__device__ __forceinline__ void dot4_range(const uint8_t* __restrict__ tile, int b0, int b1, const QAct& act,
                                           int lane, float (&acc)[T]) {
  if (b0 >= b1) return;
  Unit u0;
  load_unit(tile + (size_t)b0 * kUnitBytes, lane, u0);
  dot4_range_from<T>(tile, b0, b1, act, lane, acc, u0);
}

// Matrix-core engine (any T <= 16): v_mfma_i32_16x16x32_i8 with the
// activation rows as the 16 x 32 A operand (rows t >= T are zero) and one
// 16-row group of weights x one sub-block as the 32 x 16 B operand.  Lane
// l = 16*kq + nl holds A[t = nl][k = 8kq..8kq+7], B[k = 8kq..8kq+7][n = nl]
// and the result C[t = 4kq + i][n = nl], i = 0..3.  One wave covers the 4
// groups (64 rows) of a tile; acc[grp][i] is output row 16*grp + nl, row t = 4kq + i.
struct UnitM {
  u32x4 h[4];      // header of row 16*grp + nl
  uint32_t c[4][8]; // dword kq of (row 16*grp + nl, sub-block j)
};


// A unit loaded with lane = row (load_unit) into the matrix-core operand
// layout, through the wave's LDS area ar (kUnitBytes): the unit is written in
// its global byte layout, then lane 16*kq + nl reads the headers of rows
// 16*grp + nl and dword kq of their codes.  LDS operations of one wave
// complete in order, so a later call's writes never pass these reads.
__device__ __forceinline__ void transpose_unit(const Unit& u, uint8_t* ar, int nl, int kq, int lane, UnitM& x) {
  *(u32x4*)(ar + lane * 16) = u.h;
#pragma unroll
  for (int j = 0; j < 8; ++j) *(u32x4*)(ar + kHdrBytes + j * kSubBytes + lane * 16) = u.c[j];
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) x.h[grp] = *(const u32x4*)(ar + (16 * grp + nl) * 16);
#pragma unroll
  for (int grp = 0; grp < 4; ++grp)
#pragma unroll
    for (int j = 0; j < 8; ++j) x.c[grp][j] = *(const uint32_t*)(ar + kHdrBytes + j * kSubBytes + (16 * grp + nl) * 16 + kq * 4);
}

// Activation rows of one superblock in the matrix-core operand order, as the
// engine reads them from LDS (kActSbBytes per superblock b):
//   [0, 4096)     A operand of sub-block j at j*512: lane 16*kq + t holds
//                 a8[t][256b + 32j + 8kq .. +7] (zeros for t >= T)
//   [4096, 5120)  (s, s*gsum) of group 8b + j for rows t = 0..15: float2 at
//                 4096 + (16j + t) * 8
constexpr int kActSbBytes = 5120;

// Stages superblocks [lo, lo + n) of the quantized rows into LDS in that
// layout; every thread of the 256-thread block takes part.
__device__ __forceinline__ void stage_act(const QAct& act, int lo, int n, uint8_t* lds) {
  for (int i = threadIdx.x; i < n * 512; i += 256) {
    const int sb = i >> 9, j = (i >> 6) & 7, kq = (i >> 4) & 3, t = i & 15;
    uint2 v = make_uint2(0u, 0u);
    if (t < act.T) v = *(const uint2*)(act.a8 + (size_t)t * act.K + (size_t)(lo + sb) * 256 + j * 32 + kq * 8);
    *(uint2*)(lds + sb * kActSbBytes + j * 512 + (16 * kq + t) * 8) = v;
  }
  for (int i = threadIdx.x; i < n * 64; i += 256) {
    const int sb = i >> 6, q = i & 63;
    *(u32x4*)(lds + sb * kActSbBytes + 4096 + q * 16) =
        *(const u32x4*)((const uint8_t*)act.ssg + (size_t)(lo + sb) * 1024 + q * 16);
  }
}

// One unit against the staged activation rows of its superblock (act, LDS).
// The activation reads are LDS reads, so they never wait behind the next
// unit's global loads.
__device__ __forceinline__ void mfma_unit(const UnitM& x, const uint8_t* act, int nl, int kq, float (&acc)[4][4]) {
  Hdr hd[4];
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) decode_hdr(x.h[grp], hd[grp]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const long aop = *(const long*)(act + j * 512 + (16 * kq + nl) * 8);
    const f32x4 s01 = *(const f32x4*)(act + 4096 + (16 * j + 4 * kq) * 8);
    const f32x4 s23 = *(const f32x4*)(act + 4096 + (16 * j + 4 * kq + 2) * 8);
    const float sv[4] = {s01.x, s01.z, s23.x, s23.z};
    const float sg[4] = {s01.y, s01.w, s23.y, s23.w};
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const uint32_t w = x.c[grp][j];
      const long bop = (long)(w & 0x0F0F0F0Fu) | ((long)((w >> 4) & 0x0F0F0F0Fu) << 32);
      const i32x4 z = {0, 0, 0, 0};
      const i32x4 c = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop, z, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[grp][i] = __builtin_fmaf((float)c[i] * hd[grp].dsc[j], sv[i], acc[grp][i]);
        acc[grp][i] = __builtin_fmaf(-hd[grp].dm[j], sg[i], acc[grp][i]);
      }
    }
  }
}

}  // namespace mk

namespace mk {

// Per-32 quantization of one group held by 32 consecutive lanes (lane & 31 =
// element).  s = amax/127 by IEEE division (0 for an all-zero group),
// a8 = clamp(rne(x/s), -127, 127), gsum = sum of a8 over the group.
struct Q8 {
  int a8;
  float s;
  int gsum;
};

// Cross-lane reduction steps on the VALU (DPP and the gfx950 row swaps)
// rather than LDS permutes.  The two quad permutes make each group of 4
// lanes uniform; the half-row and row mirrors then pair every lane with the
// other half of its 8- and 16-lane group; the row swaps pair 16-lane rows
// and 32-lane halves.  Every lane of a reduced group ends with the same
// value, combined in the same order.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
// (row 2r, row 2r + 1) values of a 16-lane row pair, in every lane of both rows
__device__ __forceinline__ void rows16(float v, float& lo, float& hi) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  lo = __builtin_bit_cast(float, (unsigned)p[0]);
  hi = __builtin_bit_cast(float, (unsigned)p[1]);
}
// (lanes 0..31, lanes 32..63) values, in every lane
__device__ __forceinline__ void halves32(float v, float& lo, float& hi) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  lo = __builtin_bit_cast(float, (unsigned)p[0]);
  hi = __builtin_bit_cast(float, (unsigned)p[1]);
}
__device__ __forceinline__ float max32(float v) {
  v = __builtin_fmaxf(v, dpp_f<0xB1>(v));   // lane ^ 1
  v = __builtin_fmaxf(v, dpp_f<0x4E>(v));   // lane ^ 2
  v = __builtin_fmaxf(v, dpp_f<0x141>(v));  // half-row mirror
  v = __builtin_fmaxf(v, dpp_f<0x140>(v));  // row mirror
  float lo, hi;
  rows16(v, lo, hi);
  return __builtin_fmaxf(lo, hi);
}
__device__ __forceinline__ int sum32_i(int v) {
  v += dpp_i<0xB1>(v);
  v += dpp_i<0x4E>(v);
  v += dpp_i<0x141>(v);
  v += dpp_i<0x140>(v);
  float lo, hi;
  rows16(__builtin_bit_cast(float, v), lo, hi);
  return __builtin_bit_cast(int, lo) + __builtin_bit_cast(int, hi);
}
__device__ __forceinline__ float sum64(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  float lo, hi;
  rows16(v, lo, hi);
  v = lo + hi;
  halves32(v, lo, hi);
  return lo + hi;
}
__device__ __forceinline__ int sum64_i(int v) {
  const int s32 = sum32_i(v);
  float lo, hi;
  halves32(__builtin_bit_cast(float, s32), lo, hi);
  return __builtin_bit_cast(int, lo) + __builtin_bit_cast(int, hi);
}

__device__ __forceinline__ Q8 quant_group32(float x) {
  // amax over the group's non-NaN lanes (fmax drops a NaN operand)
  const float amax = max32(__builtin_fabsf(x));
  const float s = amax / 127.0f;
  Q8 r;
  if (!(s > 0.0f)) {
    // an all-zero group, a scale that underflows, or a group of NaN only
    r.s = 0.0f;
    r.a8 = 0;
  } else {
    r.s = s;
    const float q = __builtin_rintf(x / s);
    // a NaN quotient (a NaN element, or inf / inf) codes as 0
    r.a8 = q == q ? (int)__builtin_fminf(__builtin_fmaxf(q, -127.0f), 127.0f) : 0;
  }
  r.gsum = sum32_i(r.a8);
  return r;
}

}  // namespace mk
