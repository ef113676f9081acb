// mk_lm.h — the lm_head stream shared by the standalone lm_head + verify
// kernel and the lm phase of the decode step (pages: richland.au
// single-stream article, "What shipped" — lm_head and verification run on
// the device and the host reads back only the accepted tokens).
//
// logits[t][v] = sum_h f32(W[v][h]) * hid[t][h] on the fp16 matrix cores:
// hid is pre-split into hi = fp16(hid) and lo = fp16(hid - hi) fragments and
// both halves are multiplied against the same weight fragment with fp32
// accumulation (a product of two fp16 values is exact in fp32).  Block b
// takes the vocabulary rows of 16-row groups [G*b/n, G*(b+1)/n) (G = V/16
// rounded up, n blocks), in 64-row chunks; its NW waves split the 64-wide
// hidden chunks of each, and every wave keeps the loads of its next two
// items in flight while its MFMAs run, across chunk boundaries.
#pragma once
#include "mk_device.h"

namespace mk {

struct LmStream {
  const uint16_t* W;     // [V][H] fp16 bits, row-major
  const _Float16* frag;  // [H/64][64 lanes][hi 16 | lo 16]: lane 16*kq + t holds h = 64c + 16kq + e of row t
  int V, H;
  float* val;        // [gridDim.x][16] per-block winners (value)
  int* idx;          // [gridDim.x][16] per-block winners (vocabulary index)
  unsigned* ticket;  // arrival counter; zero when the launch starts
  float* logits;     // optional [logits_T][V] output of every logit (null: none)
  int logits_T;      // rows of `logits` (rows t < logits_T are stored)
};

// One 64-wide hidden chunk of 64 vocabulary rows: the weight fragments of
// the 4 row groups of 16 and the hi/lo fragments of the hidden rows.
struct LmChunk {
  u32x4 wa[4][2];
  u32x4 bh0, bh1, bl0, bl1;
};

// rows v0 .. v0 + 63 (clamped below rhi), hidden chunk c
__device__ __forceinline__ void lm_load(const LmStream& a, int v0, int rhi, int c, int l, int vl, int kq,
                                        LmChunk& x) {
  const u32x4* fp = (const u32x4*)(a.frag + ((size_t)c * 64 + l) * 32);
  x.bh0 = fp[0];
  x.bh1 = fp[1];
  x.bl0 = fp[2];
  x.bl1 = fp[3];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int v = v0 + 16 * g + vl;
    const int vv = v < rhi ? v : rhi - 1;  // a row of the block's range; results of rows >= rhi are never used
    // cached loads: the two half-line loads of a row merge in L2
    const u32x4* wpp = (const u32x4*)(a.W + (size_t)vv * a.H + 64 * c + 16 * kq);
    x.wa[g][0] = wpp[0];
    x.wa[g][1] = wpp[1];
  }
}

__device__ __forceinline__ void lm_mfma(const LmChunk& x, f32x4 (&acc)[4]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x.wa[g][0]),
                                                    __builtin_bit_cast(f16x8, x.bh0), acc[g], 0, 0, 0);
    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x.wa[g][0]),
                                                    __builtin_bit_cast(f16x8, x.bl0), acc[g], 0, 0, 0);
    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x.wa[g][1]),
                                                    __builtin_bit_cast(f16x8, x.bh1), acc[g], 0, 0, 0);
    acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x.wa[g][1]),
                                                    __builtin_bit_cast(f16x8, x.bl1), acc[g], 0, 0, 0);
  }
}

// (value, index) order of the argmax: the larger value wins, then the lower
// index; index -1 means "no candidate".  A NaN candidate never wins, not even
// over "no candidate", so a row whose logits are all NaN keeps index -1.
__device__ __forceinline__ bool lm_better(float va, int ia, float vb, int ib) {
  if (ia < 0 || va != va) return false;
  if (ib < 0 || vb != vb) return true;
  return va > vb || (va == vb && ia < ib);
}

// Streams the block's vocabulary rows with all NW waves of the block; red is
// NW x 64 x 16 floats of LDS.  Returns true in the last block to arrive,
// whose fin[t] (t < 16, LDS) then holds the argmax of row t over the whole
// vocabulary (-1 where no row was seen); returns false in every other block.
// Every thread of the block must call it.
template <int NW>
__device__ __forceinline__ bool lm_stream(const LmStream& a, float (*red)[64][16], int* fin) {
  constexpr int TPT = 16;  // threads per row t in the scans (the block's first 256 threads)
  __shared__ int last;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int vl = l & 15, kq = l >> 4;
  const int nc = a.H / 64;
  const int c0 = (nc * w) / NW, nck = (nc * (w + 1)) / NW - c0;  // the wave's hidden chunks
  const int M = (nc + NW - 1) / NW;  // items per 64-row chunk, the same for every wave
  const int ng = (a.V + 15) / 16;
  const int g0 = (int)((long)ng * blockIdx.x / gridDim.x), g1 = (int)((long)ng * (blockIdx.x + 1) / gridDim.x);
  const int rlo = 16 * g0, rhi = 16 * g1 < a.V ? 16 * g1 : a.V;  // the block's vocabulary rows
  const int nb = (g1 - g0 + 3) / 4;                            // its 64-row chunks
  const int n = nb * M;                                        // the wave's items (chunk k, slot cc)
  const bool scan = threadIdx.x < 16 * TPT;  // threads that scan: row t_own, every TPT-th vocabulary row
  const int t_own = scan ? threadIdx.x / TPT : 0, part = threadIdx.x % TPT;
  float best = 0.0f;
  int bidx = -1;
  // Item (k, cc) is hidden chunk c0 + cc of rows rlo + 64k ..; slots
  // cc >= nck (waves with fewer chunks) re-read the wave's last chunk and are
  // not multiplied, so that every wave passes the same chunk boundaries.
  int kn = 0, cn = 0;  // the next item to load; past the last item, the last one again
  auto load_next = [&](LmChunk& x) {
    const int c = nck > 0 ? c0 + (cn < nck ? cn : nck - 1) : (c0 < nc ? c0 : nc - 1);
    lm_load(a, rlo + 64 * kn, rhi, c, l, vl, kq, x);
    if (++cn == M) {
      if (kn + 1 < nb) {
        cn = 0;
        ++kn;
      } else {
        cn = M - 1;
      }
    }
  };
  f32x4 acc[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) acc[g] = (f32x4){0.f, 0.f, 0.f, 0.f};
  int k = 0, cc = 0;  // the item being multiplied
  // multiply the current item; after the last item of a chunk, reduce the
  // waves' sums through LDS and scan the chunk's rows
  auto consume = [&](const LmChunk& x) {
    if (cc < nck) lm_mfma(x, acc);
    if (++cc == M) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[w][16 * g + 4 * kq + i][vl] = acc[g][i];  // C[v = 16g + 4kq + i][t = vl]
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[g] = (f32x4){0.f, 0.f, 0.f, 0.f};
      __syncthreads();
      const int v0 = rlo + 64 * k;
      for (int r = part; r < 64 && scan; r += TPT) {
        const int v = v0 + r;
        if (v >= rhi) break;
        float xv = red[0][r][t_own];
#pragma unroll
        for (int q = 1; q < NW; ++q) xv += red[q][r][t_own];
        if (a.logits && t_own < a.logits_T) a.logits[(size_t)t_own * a.V + v] = xv;
        if (lm_better(xv, v, best, bidx)) {
          best = xv;
          bidx = v;
        }
      }
      __syncthreads();
      cc = 0;
      ++k;
    }
  };
  // Three buffers in rotation: the loads are unconditional and the
  // scheduling barriers pin their position, so each buffer keeps its
  // registers and two items are always in flight.
  if (n > 0) {
    LmChunk b0, b1, b2;
    load_next(b0);
    load_next(b1);
    for (int i = 0; i < n; i += 3) {
      load_next(b2);
      __builtin_amdgcn_sched_barrier(0);
      consume(b0);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 >= n) break;
      load_next(b0);
      __builtin_amdgcn_sched_barrier(0);
      consume(b1);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 2 >= n) break;
      load_next(b1);
      __builtin_amdgcn_sched_barrier(0);
      consume(b2);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int m = TPT / 2; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(best, m, TPT);
    const int oi = __shfl_xor(bidx, m, TPT);
    if (lm_better(ov, oi, best, bidx)) {
      best = ov;
      bidx = oi;
    }
  }
  if (scan && part == 0) {
    st_coh(a.val + (size_t)blockIdx.x * 16 + t_own, best);
    st_coh((float*)a.idx + (size_t)blockIdx.x * 16 + t_own, __builtin_bit_cast(float, bidx));
  }
  stores_done();  // every wave's stores are in memory before thread 0 takes the ticket
  __syncthreads();
  if (threadIdx.x == 0) last = (ticket_add(a.ticket) == gridDim.x - 1);
  __syncthreads();
  if (!last) return false;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  best = 0.0f;
  bidx = -1;
  for (int b = part; b < (int)gridDim.x && scan; b += TPT) {
    const float xv = ld_coh(a.val + (size_t)b * 16 + t_own);
    const int iv = ld_coh_i(a.idx + (size_t)b * 16 + t_own);
    if (lm_better(xv, iv, best, bidx)) {
      best = xv;
      bidx = iv;
    }
  }
#pragma unroll
  for (int m = TPT / 2; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(best, m, TPT);
    const int oi = __shfl_xor(bidx, m, TPT);
    if (lm_better(ov, oi, best, bidx)) {
      best = ov;
      bidx = oi;
    }
  }
  if (scan && part == 0) fin[t_own] = bidx;
  __syncthreads();
  return true;
}


// ---------------------------------------------------------------------------
// The same stream with the weights staged through LDS: each 1-KB segment of
// a vocabulary row (512 hidden values) arrives by one LDS-DMA load (64 lanes
// x 16 contiguous bytes of one row), and the matrix-core operands are read
// back from LDS.  Loads that each cover one row run read HBM faster than
// loads that touch 16 rows at once.  A stage is 32 rows x one segment (rows
// 1040 B apart in LDS, so that the 16 rows of an operand read fall on
// different banks); NS stages rotate, NS - 1 in flight.  Wave w of the 8
// multiplies hidden chunk 8 s + w of every segment s, and keeps the
// fragments of its chunks in registers for the whole stream, so that the
// only vector-memory operations it waits for are its stage loads.  Needs
// H = 512 NSEG.  stages: NS x kLmStageBytes of LDS; the
// cross-wave sums of a finished 32-row chunk go to the stage buffer that is
// free at that point.
constexpr int kLmRows = 32;                       // rows per stage
constexpr int kLmRowStride = 1040;                // LDS bytes per staged row
constexpr int kLmStageBytes = kLmRows * kLmRowStride;

__device__ __forceinline__ void lm_stage_dma(uint32_t lds_row0, const uint16_t* W, int H, int seg, int r0, int rhi,
                                             int w, int lane) {
  // wave w loads rows 4w .. 4w + 3 of the stage
#pragma unroll
  for (int i = 0; i < kLmRows / 8; ++i) {
    const int rr = 4 * w + i, v = r0 + rr < rhi ? r0 + rr : rhi - 1;  // rows past the range re-read a valid row
    const uint64_t g = (uint64_t)(uintptr_t)(W + (size_t)v * H + 512 * seg) + 16 * lane;
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds_row0 + rr * kLmRowStride);
    asm volatile("s_mov_b32 m0, %[m]\n\tglobal_load_lds_dwordx4 %[a], off" : : [a] "v"(g), [m] "s"(m) : "memory", "m0");
  }
}

template <int NS, int NSEG>
__device__ __forceinline__ bool lm_stream_staged(const LmStream& a, uint8_t* stages, int* fin) {
  constexpr int NW = 8, TPT = 16, NB = kLmRows / 16, NCH = NSEG;
  static_assert(NS >= 2 && NS <= 4, "two to four stages");
  static_assert(NW * kLmRows * 16 * 4 <= kLmStageBytes, "the sums fit a stage buffer");
  __shared__ int last;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int vl = l & 15, kq = l >> 4;
  constexpr int nseg = NSEG;  // a.H == 512 * NSEG
  // the wave's fragments: chunk c = 8 s + w
  u32x4 fr[NCH][4];
#pragma unroll
  for (int s = 0; s < NCH; ++s) {
    const u32x4* fp = (const u32x4*)(a.frag + ((size_t)(8 * s + w) * 64 + l) * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) fr[s][i] = fp[i];
  }
  const int ng = (a.V + 15) / 16;
  const int g0 = (int)((long)ng * blockIdx.x / gridDim.x), g1 = (int)((long)ng * (blockIdx.x + 1) / gridDim.x);
  const int rlo = 16 * g0, rhi = 16 * g1 < a.V ? 16 * g1 : a.V;
  const int nchunk = (g1 - g0 + NB - 1) / NB;
  const int n = nchunk * nseg;  // stages: i = chunk k * nseg + segment s
  const bool scan = threadIdx.x < 16 * TPT;
  const int t_own = scan ? threadIdx.x / TPT : 0, part = threadIdx.x % TPT;
  float best = 0.0f;
  int bidx = -1;
  const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)stages;
  // the next stage to load: its buffer, segment and first row (past the
  // end: the last stage again); advanced without divisions
  int ib = 0, is = 0, ir = rlo, left = n;
  auto issue = [&]() {
    lm_stage_dma(base + (uint32_t)ib * kLmStageBytes, a.W, a.H, is, ir, rhi, w, l);
    ib = ib + 1 == NS ? 0 : ib + 1;
    if (--left > 0) {
      if (++is == nseg) {
        is = 0;
        ir += kLmRows;
      }
    }
  };
  f32x4 acc[NB];
#pragma unroll
  for (int g = 0; g < NB; ++g) acc[g] = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (n > 0) {
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) issue();
  }
  int cb = 0;  // buffer of the next stage to multiply
  for (int k = 0; k < nchunk; ++k) {
    uint8_t* sb = stages;
#pragma unroll
    for (int s = 0; s < NCH; ++s) {  // unrolled: the fragment registers are indexed statically
      {
        // this wave's loads of stage i are done when at most the later stages' are in flight
        static_assert(kLmRows / 8 == 4, "four loads per wave and stage");
        if constexpr (NS == 4)
          asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else if constexpr (NS == 3)
          asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // every wave's loads of stage i have landed; every wave is done with stage i - 1
        issue();
        typedef __attribute__((address_space(3))) const u32x4 lds_v;
        sb = stages + cb * kLmStageBytes;
        cb = cb + 1 == NS ? 0 : cb + 1;
#pragma unroll
        for (int g = 0; g < NB; ++g) {
          const uint8_t* rp = sb + (16 * g + vl) * kLmRowStride + (64 * w + 16 * kq) * 2;
          const u32x4 w0 = *(lds_v*)rp, w1 = *(lds_v*)(rp + 16);
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, w0),
                                                          __builtin_bit_cast(f16x8, fr[s][0]), acc[g], 0, 0, 0);
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, w0),
                                                          __builtin_bit_cast(f16x8, fr[s][2]), acc[g], 0, 0, 0);
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, w1),
                                                          __builtin_bit_cast(f16x8, fr[s][1]), acc[g], 0, 0, 0);
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, w1),
                                                          __builtin_bit_cast(f16x8, fr[s][3]), acc[g], 0, 0, 0);
        }
      }
    }
    // The chunk's rows are complete: reduce over the waves and scan.  The
    // sums go to the buffer of the chunk's last stage: no load targets it
    // until after the next stage's barrier, and every wave has read its
    // operands from it (the barrier below follows every wave's reads).
    __syncthreads();
    float(*red)[kLmRows][16] = (float(*)[kLmRows][16])sb;
#pragma unroll
    for (int g = 0; g < NB; ++g)
#pragma unroll
      for (int q = 0; q < 4; ++q) red[w][16 * g + 4 * kq + q][vl] = acc[g][q];
#pragma unroll
    for (int g = 0; g < NB; ++g) acc[g] = (f32x4){0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    const int v0 = rlo + kLmRows * k;
    for (int r = part; r < kLmRows && scan; r += TPT) {
      const int v = v0 + r;
      if (v >= rhi) break;
      float xv = red[0][r][t_own];
#pragma unroll
      for (int q = 1; q < NW; ++q) xv += red[q][r][t_own];
      if (a.logits && t_own < a.logits_T) a.logits[(size_t)t_own * a.V + v] = xv;
      if (lm_better(xv, v, best, bidx)) {
        best = xv;
        bidx = v;
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the loads issued past the end
#pragma unroll
  for (int m = TPT / 2; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(best, m, TPT);
    const int oi = __shfl_xor(bidx, m, TPT);
    if (lm_better(ov, oi, best, bidx)) {
      best = ov;
      bidx = oi;
    }
  }
  if (scan && part == 0) {
    st_coh(a.val + (size_t)blockIdx.x * 16 + t_own, best);
    st_coh((float*)a.idx + (size_t)blockIdx.x * 16 + t_own, __builtin_bit_cast(float, bidx));
  }
  stores_done();  // every wave's stores are in memory before thread 0 takes the ticket
  __syncthreads();
  if (threadIdx.x == 0) last = (ticket_add(a.ticket) == gridDim.x - 1);
  __syncthreads();
  if (!last) return false;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  best = 0.0f;
  bidx = -1;
  for (int b = part; b < (int)gridDim.x && scan; b += TPT) {
    const float xv = ld_coh(a.val + (size_t)b * 16 + t_own);
    const int iv = ld_coh_i(a.idx + (size_t)b * 16 + t_own);
    if (lm_better(xv, iv, best, bidx)) {
      best = xv;
      bidx = iv;
    }
  }
#pragma unroll
  for (int m = TPT / 2; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(best, m, TPT);
    const int oi = __shfl_xor(bidx, m, TPT);
    if (lm_better(ov, oi, best, bidx)) {
      best = ov;
      bidx = oi;
    }
  }
  if (scan && part == 0) fin[t_own] = bidx;
  __syncthreads();
  return true;
}

}  // namespace mk
