// mk_attn.h — device code of split-K flash decoding shared by the standalone
// attention launches (mk_attn.hip) and the persistent step's attention items
// (page: richland.au single-stream article, "What shipped": the attention
// layers decode with split-K flash decoding over the KV cache, matrix-core
// products on K/V tiles).  The layout of the products and the precision are
// described at the top of mk_attn.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace mk {
namespace attn {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kTile = 64;

__device__ __forceinline__ h8 as_h8(u4 u) { return __builtin_bit_cast(h8, u); }
__device__ __forceinline__ u4 as_u4(h8 h) { return __builtin_bit_cast(u4, h); }

__device__ __forceinline__ f4 mma(u4 a, u4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(a), as_h8(b), c, 0, 0, 0);
}

// x = hi + lo with hi, lo fp16.  The residual is taken from the packed hi
// bits themselves: the compiler may round the packing conversion and a
// separate scalar conversion of the same value differently on exact ties,
// and a residual from the other hi would then add the wrong sign.
__device__ __forceinline__ void split_f16(const float (&x)[8], u4& hi_out, u4& lo_out) {
  h8 hi;
#pragma unroll
  for (int j = 0; j < 8; ++j) hi[j] = (_Float16)x[j];
  u4 hb = as_u4(hi);
  asm volatile("" : "+v"(hb));
  const h8 hr = as_h8(hb);
  h8 lo;
#pragma unroll
  for (int j = 0; j < 8; ++j) lo[j] = (_Float16)(x[j] - (float)hr[j]);
  hi_out = hb;
  lo_out = as_u4(lo);
}

// Eight q8_0 codes (two dwords of int8) -> eight fp16 values, exactly: each
// byte, sign-flipped to c + 128, becomes the low byte of the fp16 1024 + c + 128
// (exponent byte 0x64), and 1152 is subtracted in packed fp16.  (Leaving the
// 1152 in and removing 1152 times the other operand's block sum afterwards
// saves the subtraction, but the cancellation costs about seven bits of the
// fp32 products.)
// The empty asm keeps each conversion at its use: with several column
// blocks the compiler would otherwise hold every converted operand of the
// tile at once and spill.
__device__ __forceinline__ u4 codes_f16(uint2 c) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  asm volatile("" : "+v"(c));
  const unsigned x0 = c.x ^ 0x80808080u, x1 = c.y ^ 0x80808080u;
  const h2 off = {(_Float16)1152.f, (_Float16)1152.f};
  u4 r;
  r[0] = __builtin_bit_cast(unsigned, __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u)) - off);
  r[1] = __builtin_bit_cast(unsigned, __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u)) - off);
  r[2] = __builtin_bit_cast(unsigned, __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u)) - off);
  r[3] = __builtin_bit_cast(unsigned, __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u)) - off);
  return r;
}

// One (agent, KV head) of the cache, in the format in use (the other
// format's pointers are null).
struct KVHead {
  const uint16_t* K;   // fp16 [cap][128], position-major
  const uint16_t* V;   // fp16 [128][cap], dimension-major
  const int8_t* K8;    // q8_0 codes [cap][128]
  const int8_t* V8;    //            [cap/64][128][64], tile-major
  const uint16_t* KS;  // q8_0 K scales [cap][4]
  const uint16_t* VS;  // q8_0 V scales [cap/32][128]
  int cap;
};

// The K and V operands of one 64-position tile.
struct KVTile {
  u4 kr[4][4], vr[2][8];     // fp16 operands
  uint2 k8[4][4], v8[2][8];  // Q8: codes
  u4 ksc[4][2];              // Q8: K scales [b][row i / 2] -> halves (i % 2) * 4 + m
  uint2 vsc[2][8];           // Q8: V scales of dims 16db + 4grp .. +3, block t0/32 + hh
};

// V positions at or past L_g contribute nothing.  In the fp16 cache they may
// hold any bits (inf or NaN times a zero probability is NaN); q8_0 codes
// always convert to finite values, so that format needs no masking.
__device__ __forceinline__ u4 zero_tail(u4 r, int t0, int hh, int grp, int Lg) {
  h8 v = as_h8(r);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (t0 + 32 * hh + 8 * grp + j >= Lg) v[j] = (_Float16)0.f;
  return as_u4(v);
}

// Loads tile t0 (a multiple of 64 below L_g <= cap, cap % 64 == 0, so every
// load stays inside the head's cache rows).  Each load is a wave-uniform base
// (the tile, the row block, the dimension block) plus one 32-bit byte offset
// per lane, so that the tile's 32 loads share two lane offsets instead of
// holding a 64-bit address each.
template <bool Q8>
__device__ __forceinline__ void load_tile(const KVHead& c, int t0, int Lg, int col, int grp, KVTile& x) {
  // lane offsets: K row 8 (col / 4) + col % 4 of the row block, dims 8 grp..;
  // V row (dimension) col of the dimension block, positions 8 grp..
  const uint32_t krow = 8 * (col >> 2) + (col & 3);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int r0 = t0 + 32 * (b >> 1) + 4 * (b & 1);  // the row block's first position (uniform)
    if constexpr (Q8) {
      const char* kb = (const char*)(c.K8 + (size_t)r0 * kD);
      const uint32_t kl = krow * kD + 8 * grp;
#pragma unroll
      for (int m = 0; m < 4; ++m) x.k8[b][m] = *(const uint2*)(kb + kl + 32 * m);
      const char* sb = (const char*)(c.KS + (size_t)r0 * (kD / 32));
      const uint32_t sl = 8 * grp * (kD / 32) * 2;
      x.ksc[b][0] = *(const u4*)(sb + sl);
      x.ksc[b][1] = *(const u4*)(sb + sl + 16);
    } else {
      const char* kb = (const char*)(c.K + (size_t)r0 * kD);
      const uint32_t kl = (krow * kD + 8 * grp) * 2;
#pragma unroll
      for (int m = 0; m < 4; ++m) x.kr[b][m] = *(const u4*)(kb + kl + 64 * m);
    }
  }
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    if constexpr (Q8) {
      const char* vb = (const char*)(c.V8 + ((size_t)(t0 >> 6) * kD + 16 * db) * kTile);
      const uint32_t vl = col * kTile + 8 * grp;
      const char* sb = (const char*)(c.VS + (size_t)(t0 >> 5) * kD + 16 * db);
      const uint32_t sl = 8 * grp;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        x.v8[hh][db] = *(const uint2*)(vb + vl + 32 * hh);
        x.vsc[hh][db] = *(const uint2*)(sb + sl + hh * kD * 2);
      }
    } else {
      const char* vb = (const char*)(c.V + (size_t)16 * db * c.cap + t0);
      const uint32_t vl = ((uint32_t)col * (uint32_t)c.cap + 8 * grp) * 2;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) x.vr[hh][db] = *(const u4*)(vb + vl + 64 * hh);
    }
  }
  if constexpr (!Q8) {
    if (t0 + kTile > Lg) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < 8; ++db) x.vr[hh][db] = zero_tail(x.vr[hh][db], t0, hh, grp, Lg);
    }
  }
}

// One pass over a loaded tile for NF column blocks at once, so that each
// q8_0 code is converted once for all of them.  For column block f: the
// scores of this lane's column (positions below lim[f] visible), the online
// softmax (running max mrow[f], this lane's share of the sum lsum[f]) and the
// P.V update of acc[f].  Each block's arithmetic, and its order, is the same
// for every NF.
template <bool Q8, int NF>
__device__ __forceinline__ void tile_update_n(const KVTile& x, int t0, int Lg, const int* lim, int grp,
                                              const u4 (*qh)[4], const u4 (*ql)[4], f4 (*acc)[8], float* mrow,
                                              float* lsum) {
  f4 sc[NF][4];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int b = 0; b < 4; ++b) sc[f][b] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if constexpr (Q8) {
        const u4 kf = codes_f16(x.k8[b][m]);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          f4 t = mma(kf, qh[f][m], f4{0.f, 0.f, 0.f, 0.f});
          t = mma(kf, ql[f][m], t);
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[f][b][i] += (float)as_h8(x.ksc[b][i >> 1])[(i & 1) * 4 + m] * t[i];
        }
      } else {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          sc[f][b] = mma(x.kr[b][m], qh[f][m], sc[f][b]);
          sc[f][b] = mma(x.kr[b][m], ql[f][m], sc[f][b]);
        }
      }
    }
  }
  u4 ph[NF][2], pl[NF][2];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    float tmax = -INFINITY;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = t0 + 32 * (b >> 1) + 8 * grp + 4 * (b & 1) + i;
        const float v = pos < lim[f] ? sc[f][b][i] : -INFINITY;
        sc[f][b][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mnew = fmaxf(mrow[f], tmax);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = exp2f(mrow[f] - muse);
    mrow[f] = mnew;
    float ps = 0.f;
    float pv[2][8];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(sc[f][b][i] - muse);
        ps += p;
        pv[b >> 1][4 * (b & 1) + i] = p;
      }
    split_f16(pv[0], ph[f][0], pl[f][0]);
    split_f16(pv[1], ph[f][1], pl[f][1]);
    lsum[f] = lsum[f] * alpha + ps;
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[f][db] *= alpha;
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      if constexpr (Q8) {
        const u4 vo = codes_f16(x.v8[hh][db]);
        // a block holding no position of this agent may carry any scale
        const bool live = t0 + 32 * hh < Lg;
        const uint2 sv = live ? x.vsc[hh][db] : make_uint2(0u, 0u);
        const h8 s8 = as_h8(u4{sv.x, sv.y, 0u, 0u});
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          f4 t = mma(vo, ph[f][hh], f4{0.f, 0.f, 0.f, 0.f});
          t = mma(vo, pl[f][hh], t);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[f][db][i] = __builtin_fmaf((float)s8[i], t[i], acc[f][db][i]);
        }
      } else {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          acc[f][db] = mma(x.vr[hh][db], ph[f][hh], acc[f][db]);
          acc[f][db] = mma(x.vr[hh][db], pl[f][hh], acc[f][db]);
        }
      }
    }
}

// One column block's pass over a loaded tile.
template <bool Q8>
__device__ __forceinline__ void tile_update(const KVTile& x, int t0, int Lg, int lim, int grp, const u4 (&qh)[4],
                                            const u4 (&ql)[4], f4 (&acc)[8], float& mrow, float& lsum) {
  tile_update_n<Q8, 1>(x, t0, Lg, &lim, grp, &qh, &ql, &acc, &mrow, &lsum);
}

}  // namespace attn
}  // namespace mk
