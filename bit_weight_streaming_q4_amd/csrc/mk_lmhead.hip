// mk_lmhead.hip — the standalone lm_head + verify entry point: the fp16
// lm_head stream with its argmax (mk_lm.h) fused with the greedy
// draft-accept compare (pages: richland.au single-stream article, "What
// shipped" — lm_head and verification run on the device and the host reads
// back only the accepted tokens; pulse-3k2 "UPDATE", "Decode accuracy" —
// greedy output is exactly the main model's greedy choice).
#include <algorithm>

#include "mk_device.h"
#include "mk_internal.h"
#include "mk_lm.h"

namespace mk {

// Each lm_head input row is multiplied by the power of two 2^k that brings
// its largest magnitude into [2^14, 2^15), so that the fp16 hi part never
// overflows and the lo part stays out of the fp16 subnormals for every
// element that matters.  The scaling is exact and multiplies every logit of
// the row by the same 2^k, so the argmax is unchanged; rows are accepted at
// any fp32 magnitude (a row holding inf or only zeros is left unscaled).
// One block per row t < 16 writes row_exp[t] = k (0 for t >= T); block 0 also
// clears the lm_head kernel's arrival counter.
__global__ __launch_bounds__(256) void k_lm_rowexp(const float* __restrict__ hid, int T, int H,
                                                   int* __restrict__ row_exp, unsigned* __restrict__ ticket) {
  __shared__ float wmax[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (t == 0 && tid == 0) *ticket = 0u;
  int k = 0;
  if (t < T) {
    const float* row = hid + (size_t)t * H;
    float m = 0.0f;
    if (H % 1024 == 0 && H <= 8192) {  // all of the thread's loads in flight together
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = 1024 * j < H ? *(const f32x4*)(row + 1024 * j + 4 * tid) : (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[j][e]));
    } else {
      for (int i = tid; i < H; i += 256) m = __builtin_fmaxf(m, __builtin_fabsf(row[i]));  // NaN is ignored
    }
    for (int o = 32; o >= 1; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, 64));
    if ((tid & 63) == 0) wmax[tid >> 6] = m;
    __syncthreads();
    m = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
    if (m > 0.0f && m <= 3.402823466e38f) {
      int e;
      __builtin_frexpf(m, &e);  // m = f * 2^e, f in [0.5, 1)
      k = 15 - e;
    }
  }
  if (tid == 0) row_exp[t] = k;
}

// hid [T][H] fp32, scaled by 2^row_exp[t] -> fragments [H/64][64 lanes][hi 16 | lo 16]
// fp16 for the B operand: lane l = 16*kq + t holds h = 64c + 16kq + e,
// e = 0..15 of row t (zeros for t >= T).
__global__ __launch_bounds__(64) void k_lm_prep(const float* __restrict__ hid, int T, int H,
                                                _Float16* __restrict__ frag, const int* __restrict__ row_exp) {
  const int c = blockIdx.x, l = threadIdx.x;
  const int t = l & 15, kq = l >> 4;
  const int k = row_exp[t];
  _Float16* o = frag + ((size_t)c * 64 + l) * 32;
  f32x4 v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    v[q] = t < T ? *(const f32x4*)(hid + (size_t)t * H + 64 * c + 16 * kq + 4 * q) : (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float x = __builtin_ldexpf(v[e >> 2][e & 3], k);
    const _Float16 hi = (_Float16)x;
    const _Float16 lo = (_Float16)(x - (float)hi);
    o[e] = hi;
    o[16 + e] = lo;
  }
}

struct LmArgs {
  LmStream s;
  int T, G;
  int gs[MK_LM_MAX_G + 1];
  const int32_t* drafts;
  int32_t* argmax;
  int32_t* n_acc;
  int32_t* tokens;
  int verify;  // the last block writes argmax and runs the greedy accept compare
};

constexpr int kLmWaves = 8;
#ifndef MK_LM_BLOCKS_PER_CU
#define MK_LM_BLOCKS_PER_CU 1
#endif
constexpr int kLmBlocksPerCu = MK_LM_BLOCKS_PER_CU;  // resident lm_head blocks per CU

// The last block's verification: argmax of every row and the accept compare
// of every group.
__device__ __forceinline__ void lm_verify(const LmArgs& a, const int* fin) {
  if (threadIdx.x < a.T) a.argmax[threadIdx.x] = fin[threadIdx.x];
  if (threadIdx.x == 0) {
    for (int g = 0; g < a.G; ++g) {
      const int r = a.gs[g], n = a.gs[g + 1] - a.gs[g];
      const int32_t* dr = a.drafts + (r - g);
      int acc_n = 0;
      while (acc_n < n - 1 && fin[r + acc_n] >= 0 && dr[acc_n] == fin[r + acc_n]) ++acc_n;
      a.n_acc[g] = acc_n;
      for (int i = 0; i < n; ++i) a.tokens[r + i] = i < acc_n ? dr[i] : (i == acc_n ? fin[r + acc_n] : -1);
    }
  }
}

// A persistent grid (a few blocks per CU) streams the vocabulary through
// lm_stream; the last block to finish writes the argmax of every row and
// runs the accept compare of every group.
__global__ __launch_bounds__(64 * kLmWaves) void k_lmhead(LmArgs a) {
  __shared__ float red[kLmWaves][64][16];
  __shared__ int fin[16];
  if (!lm_stream<kLmWaves>(a.s, red, fin) || !a.verify) return;
  lm_verify(a, fin);
}

// The same with the weights staged through LDS (H = 512 NSEG): one block of
// 8 waves per CU, 4 stages.
template <int NSEG>
__global__ __launch_bounds__(512) void k_lmhead_staged(LmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t stages[4 * kLmStageBytes];
  __shared__ int fin[16];
  if (!lm_stream_staged<4, NSEG>(a.s, stages, fin) || !a.verify) return;
  lm_verify(a, fin);
}

typedef void (*LmKernel)(LmArgs);
static LmKernel staged_kernel(int nseg) {
  switch (nseg) {
    case 1: return k_lmhead_staged<1>;
    case 2: return k_lmhead_staged<2>;
    case 3: return k_lmhead_staged<3>;
    case 4: return k_lmhead_staged<4>;
    case 5: return k_lmhead_staged<5>;
    case 6: return k_lmhead_staged<6>;
    case 7: return k_lmhead_staged<7>;
    case 8: return k_lmhead_staged<8>;
    case 9: return k_lmhead_staged<9>;
    case 10: return k_lmhead_staged<10>;
    default: return nullptr;  // longer rows: the register-streamed kernel
  }
}

size_t lm_frag_bytes(int H) { return (size_t)(H / 64) * 64 * 32 * sizeof(_Float16); }
int lm_nblocks(int V) { return (V + 63) / 64; }

hipError_t launch_lmhead(const uint16_t* W, int V, int H, const float* hid, int T, const int32_t* gs, int G,
                         const int32_t* drafts, int32_t* argmax, int32_t* n_acc, int32_t* tokens, void* ws,
                         int cu_count, hipStream_t st) {
  return launch_lm_stream(W, V, H, hid, T, gs, G, drafts, argmax, n_acc, tokens, ws, cu_count, st, nullptr, nullptr);
}

// The lm_head stream with the greedy verification (logits == null), or
// writing every logit to logits [T][V] (scaled rows: logit * 2^row_exp[t])
// without it.
hipError_t launch_lm_stream(const uint16_t* W, int V, int H, const float* hid, int T, const int32_t* gs, int G,
                            const int32_t* drafts, int32_t* argmax, int32_t* n_acc, int32_t* tokens, void* ws,
                            int cu_count, hipStream_t st, float* logits, int* row_exp) {
  uint8_t* p = (uint8_t*)ws;
  uint32_t* ticket = (uint32_t*)p;            // word 0 of the first 256 B
  int* rexp = row_exp ? row_exp : (int*)(p + 64);  // words 16..31 (unless the caller keeps them)
  p += 256;
  _Float16* frag = (_Float16*)p;
  p += (lm_frag_bytes(H) + 255) / 256 * 256;
  const int nblk = lm_nblocks(V);
  float* pval = (float*)p;
  p += ((size_t)nblk * 16 * 4 + 255) / 256 * 256;
  int32_t* pidx = (int32_t*)p;
  hipLaunchKernelGGL(k_lm_rowexp, dim3(16), dim3(256), 0, st, hid, T, H, rexp, ticket);
  hipLaunchKernelGGL(k_lm_prep, dim3(H / 64), dim3(64), 0, st, hid, T, H, frag, rexp);
  LmArgs a;
  a.s.W = W;
  a.s.frag = frag;
  a.s.V = V;
  a.s.H = H;
  a.s.val = pval;
  a.s.idx = pidx;
  a.s.ticket = ticket;
  a.s.logits = logits;
  a.s.logits_T = logits ? T : 0;
  a.verify = logits ? 0 : 1;
  a.T = T;
  a.G = G;
  for (int i = 0; i <= MK_LM_MAX_G; ++i) a.gs[i] = i <= G ? gs[i] : T;
  a.drafts = drafts;
  a.argmax = argmax;
  a.n_acc = n_acc;
  a.tokens = tokens;
  const LmKernel ks = H % 512 ? nullptr : staged_kernel(H / 512);
  if (ks) {
    // one block per CU (and no more blocks than the winner arrays hold)
    const int grid = std::min(nblk, cu_count);
    hipLaunchKernelGGL(ks, dim3(grid), dim3(512), 0, st, a);
  } else {
    const int grid = std::min(nblk, cu_count * kLmBlocksPerCu);
    hipLaunchKernelGGL(k_lmhead, dim3(grid), dim3(64 * kLmWaves), 0, st, a);
  }
  return hipGetLastError();
}

size_t lm_workspace_bytes(int V, int H) {
  const int nblk = lm_nblocks(V);
  return 256 + (lm_frag_bytes(H) + 255) / 256 * 256 + 2 * (((size_t)nblk * 16 * 4 + 255) / 256 * 256);
}

}  // namespace mk
