// mk_lmhead.hip — lm_head GEMV fused with a two-pass argmax and the greedy
// draft-accept compare (pages: richland.au single-stream article, "What
// shipped" — lm_head and verification run on the device and the host reads
// back only the accepted tokens; pulse-3k2 "UPDATE", "Decode accuracy" —
// greedy output is exactly the main model's greedy choice).
//
// logits[t][v] = sum_h f32(W[v][h]) * hid[t][h].  The fp16 weights are a
// dense contraction with the T hidden rows, so they go through the fp16
// matrix cores: hid (fp32) is split into hi = fp16(hid) and lo = fp16(hid - hi)
// and both halves are multiplied against the same weight fragment, with fp32
// accumulation (products of two fp16 values are exact in fp32).
#include "mk_device.h"
#include "mk_internal.h"

namespace mk {

// hid [T][H] fp32 -> fragments [H/64][64 lanes][hi 16 | lo 16] fp16 for the
// B operand: lane l = 16*kq + t holds h = 64c + 16kq + e, e = 0..15 of row t
// (zeros for t >= T).
__global__ __launch_bounds__(64) void k_lm_prep(const float* __restrict__ hid, int T, int H,
                                                _Float16* __restrict__ frag) {
  const int c = blockIdx.x, l = threadIdx.x;
  const int t = l & 15, kq = l >> 4;
  _Float16* o = frag + ((size_t)c * 64 + l) * 32;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float x = t < T ? hid[(size_t)t * H + 64 * c + 16 * kq + e] : 0.0f;
    const _Float16 hi = (_Float16)x;
    const _Float16 lo = (_Float16)(x - (float)hi);
    o[e] = hi;
    o[16 + e] = lo;
  }
}

// (value, index) order of the argmax: larger value wins, then lower index;
// NaN never wins; index -1 means "no candidate".
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  if (ia < 0) return false;
  if (ib < 0) return true;
  if (va != va) return false;
  if (vb != vb) return true;
  return va > vb || (va == vb && ia < ib);
}

struct LmArgs {
  const uint16_t* W;
  const _Float16* frag;
  int V, H, T, G;
  int gs[MK_LM_MAX_G + 1];
  const int32_t* drafts;
  int32_t* argmax;
  int32_t* n_acc;
  int32_t* tokens;
  float* pval;     // [nblk][16]
  int32_t* pidx;   // [nblk][16]
  uint32_t* ticket;
};

// Block = 4 waves on 64 vocabulary rows; wave w takes a quarter of the
// 64-wide hidden chunks for all 64 rows (4 groups of 16).  The 4 wave sums
// are added in wave order through LDS, then the block's argmax per row t is
// written; the last block to finish (atomic ticket) reduces the per-block
// winners in block order and runs the accept compare.
__global__ __launch_bounds__(256) void k_lmhead(LmArgs a) {
  __shared__ float red[4][64][16];
  __shared__ float bv[16][16];
  __shared__ int bi[16][16];
  __shared__ int last;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int vl = l & 15, kq = l >> 4;
  const int v0 = blockIdx.x * 64;
  const int nc = a.H / 64;
  const int c0 = (nc * w) / 4, c1 = (nc * (w + 1)) / 4;
  f32x4 acc[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) acc[g] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int c = c0; c < c1; ++c) {
    const u32x4* fp = (const u32x4*)(a.frag + ((size_t)c * 64 + l) * 32);
    const u32x4 bh0 = fp[0], bh1 = fp[1], bl0 = fp[2], bl1 = fp[3];
    u32x4 wa[4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int v = v0 + 16 * g + vl;
      if (v < a.V) {
        const u32x4* wp = (const u32x4*)(a.W + (size_t)v * a.H + 64 * c + 16 * kq);
        wa[g][0] = wp[0];  // cached: the two half-line loads of a row merge in L2
        wa[g][1] = wp[1];
      } else {
        wa[g][0] = (u32x4){0u, 0u, 0u, 0u};
        wa[g][1] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, wa[g][0]),
                                                      __builtin_bit_cast(f16x8, bh0), acc[g], 0, 0, 0);
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, wa[g][0]),
                                                      __builtin_bit_cast(f16x8, bl0), acc[g], 0, 0, 0);
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, wa[g][1]),
                                                      __builtin_bit_cast(f16x8, bh1), acc[g], 0, 0, 0);
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, wa[g][1]),
                                                      __builtin_bit_cast(f16x8, bl1), acc[g], 0, 0, 0);
    }
  }
  // C[v = 16g + 4kq + i][t = vl]
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w][16 * g + 4 * kq + i][vl] = acc[g][i];
  __syncthreads();
  {
    // thread (t = tid >> 4, part = tid & 15) scans rows 4*part .. 4*part+3
    const int t = threadIdx.x >> 4, part = threadIdx.x & 15;
    float best = 0.0f;
    int bidx = -1;
    for (int r = 4 * part; r < 4 * part + 4; ++r) {
      const int v = v0 + r;
      if (v >= a.V) break;
      const float x = ((red[0][r][t] + red[1][r][t]) + red[2][r][t]) + red[3][r][t];
      if (better(x, v, best, bidx)) {
        best = x;
        bidx = v;
      }
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(best, m, 16);
      const int oi = __shfl_xor(bidx, m, 16);
      if (better(ov, oi, best, bidx)) {
        best = ov;
        bidx = oi;
      }
    }
    if (part == 0) {
      a.pval[(size_t)blockIdx.x * 16 + t] = best;
      a.pidx[(size_t)blockIdx.x * 16 + t] = bidx;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const unsigned prev = atomicAdd(a.ticket, 1u);
    last = (prev == gridDim.x - 1);
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  {
    const int t = threadIdx.x >> 4, part = threadIdx.x & 15;
    float best = 0.0f;
    int bidx = -1;
    for (int b = part; b < (int)gridDim.x; b += 16) {
      const float x = __builtin_nontemporal_load(a.pval + (size_t)b * 16 + t);
      const int i = __builtin_nontemporal_load(a.pidx + (size_t)b * 16 + t);
      if (better(x, i, best, bidx)) {
        best = x;
        bidx = i;
      }
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(best, m, 16);
      const int oi = __shfl_xor(bidx, m, 16);
      if (better(ov, oi, best, bidx)) {
        best = ov;
        bidx = oi;
      }
    }
    if (part == 0) bi[0][t] = bidx;
  }
  __syncthreads();
  if (threadIdx.x < a.T) a.argmax[threadIdx.x] = bi[0][threadIdx.x];
  if (threadIdx.x == 0) {
    for (int g = 0; g < a.G; ++g) {
      const int r = a.gs[g], n = a.gs[g + 1] - a.gs[g];
      const int32_t* dr = a.drafts + (r - g);
      int acc_n = 0;
      while (acc_n < n - 1 && bi[0][r + acc_n] >= 0 && dr[acc_n] == bi[0][r + acc_n]) ++acc_n;
      a.n_acc[g] = acc_n;
      for (int i = 0; i < n; ++i) a.tokens[r + i] = i < acc_n ? dr[i] : (i == acc_n ? bi[0][r + acc_n] : -1);
    }
    *a.ticket = 0u;  // ready for the next call
  }
}

size_t lm_frag_bytes(int H) { return (size_t)(H / 64) * 64 * 32 * sizeof(_Float16); }
int lm_nblocks(int V) { return (V + 63) / 64; }

hipError_t launch_lmhead(const uint16_t* W, int V, int H, const float* hid, int T, const int32_t* gs, int G,
                         const int32_t* drafts, int32_t* argmax, int32_t* n_acc, int32_t* tokens, void* ws,
                         hipStream_t st) {
  uint8_t* p = (uint8_t*)ws;
  uint32_t* ticket = (uint32_t*)p;
  p += 256;
  _Float16* frag = (_Float16*)p;
  p += (lm_frag_bytes(H) + 255) / 256 * 256;
  const int nblk = lm_nblocks(V);
  float* pval = (float*)p;
  p += ((size_t)nblk * 16 * 4 + 255) / 256 * 256;
  int32_t* pidx = (int32_t*)p;
  hipError_t e = hipMemsetAsync(ticket, 0, 4, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_lm_prep, dim3(H / 64), dim3(64), 0, st, hid, T, H, frag);
  LmArgs a;
  a.W = W;
  a.frag = frag;
  a.V = V;
  a.H = H;
  a.T = T;
  a.G = G;
  for (int i = 0; i <= MK_LM_MAX_G; ++i) a.gs[i] = i <= G ? gs[i] : T;
  a.drafts = drafts;
  a.argmax = argmax;
  a.n_acc = n_acc;
  a.tokens = tokens;
  a.pval = pval;
  a.pidx = pidx;
  a.ticket = ticket;
  hipLaunchKernelGGL(k_lmhead, dim3(nblk), dim3(256), 0, st, a);
  return hipGetLastError();
}

size_t lm_workspace_bytes(int V, int H) {
  const int nblk = lm_nblocks(V);
  return 256 + (lm_frag_bytes(H) + 255) / 256 * 256 + 2 * (((size_t)nblk * 16 * 4 + 255) / 256 * 256);
}

}  // namespace mk
