// mk_sample.hip — sampling-mode verification: the top-k candidates of each
// row's logits, then the speculative-sampling accept / resample pass that
// keeps the target distribution (pulse-3k2, "UPDATE: ... KL divergence 0.0009
// vs llama.cpp", section "Decode accuracy vs llama.cpp": sampling keeps the
// same distribution as without drafts; top_k is capped at 32 per the
// single-stream article's "Caveats" and the 4-agent article's limits).
//
// The logits come from the lm_head stream (mk_lm.h), which writes every
// logit of rows scaled by the exact power of two 2^row_exp[t] chosen by its
// prep kernel; the scaling is monotone, so the top-k set is found on the
// scaled values and only the selected values are scaled back (exactly).
#include "mk_device.h"
#include "mk_internal.h"

namespace mk {

// Order-preserving key of a float: larger float, larger key; NaN lowest (it
// never counts as a candidate).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  if (x != x) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopKThreads = 1024;

// One block per row t: the k largest logits (ties broken towards the lower
// vocabulary index), written in ascending vocabulary order.  The k-th
// largest key is found by four 8-bit radix passes (MSB first) over the row;
// when several logits equal it, the lowest-index ones are taken by four more
// passes over their indices.  Every choice is made from exact counts, so the
// set does not depend on timing.
__global__ __launch_bounds__(kTopKThreads) void k_topk(SampleArgs a) {
  __shared__ unsigned hist[256];
  __shared__ unsigned sh_digit, sh_rem, sh_eq, sh_cnt, sh_nonnan;
  __shared__ int sel_idx[kTopKMax];
  __shared__ float sel_val[kTopKMax];
  const int t = blockIdx.x, tid = threadIdx.x;
  const float* row = a.logits + (size_t)t * a.V;
  if (tid == 0) {
    sh_cnt = 0;
    sh_nonnan = 0;
  }
  __syncthreads();
  unsigned nn = 0;
  for (int v = tid; v < a.V; v += kTopKThreads) nn += row[v] == row[v];
  if (nn) atomicAdd(&sh_nonnan, nn);
  __syncthreads();
  const unsigned keff = sh_nonnan < (unsigned)a.k ? sh_nonnan : (unsigned)a.k;
  // the keff-th largest key
  uint32_t prefix = 0, mask = 0;
  unsigned rem = keff, n_eq = 0;
  for (int p = 0; p < 4 && keff > 0; ++p) {
    const int shift = 24 - 8 * p;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int v = tid; v < a.V; v += kTopKThreads) {
      const uint32_t key = order_key(row[v]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      unsigned cum = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (cum + hist[d] >= rem) break;
        cum += hist[d];
      }
      sh_digit = (unsigned)d;
      sh_rem = rem - cum;
      sh_eq = hist[d];
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 0xFFu << shift;
    rem = sh_rem;
    n_eq = sh_eq;  // after the last pass: the number of logits whose key is exactly the threshold
    __syncthreads();
  }
  const uint32_t kth = prefix;
  // among the logits equal to the threshold, the rem lowest indices
  uint32_t iprefix = 0xFFFFFFFFu;  // every index qualifies when all ties are taken
  if (keff > 0 && n_eq > rem) {
    uint32_t ip = 0, imask = 0;
    unsigned irem = rem;
    for (int p = 0; p < 4; ++p) {
      const int shift = 24 - 8 * p;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int v = tid; v < a.V; v += kTopKThreads)
        if (order_key(row[v]) == kth && ((uint32_t)v & imask) == ip) atomicAdd(&hist[((uint32_t)v >> shift) & 255u], 1u);
      __syncthreads();
      if (tid == 0) {
        unsigned cum = 0;
        int d = 0;
        for (; d < 255; ++d) {
          if (cum + hist[d] >= irem) break;
          cum += hist[d];
        }
        sh_digit = (unsigned)d;
        sh_rem = irem - cum;
      }
      __syncthreads();
      ip |= sh_digit << shift;
      imask |= 0xFFu << shift;
      irem = sh_rem;
      __syncthreads();
    }
    iprefix = ip;  // the rem-th lowest index among the ties
  }
  if (keff > 0) {
    for (int v = tid; v < a.V; v += kTopKThreads) {
      const float x = row[v];
      const uint32_t key = order_key(x);
      if (key > kth || (key == kth && (uint32_t)v <= iprefix)) {
        const unsigned slot = atomicAdd(&sh_cnt, 1u);
        if (slot < (unsigned)kTopKMax) {
          sel_idx[slot] = v;
          sel_val[slot] = x;
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int n = sh_cnt < keff ? (int)sh_cnt : (int)keff;
    // ascending vocabulary order (at most 32 entries)
    for (int i = 1; i < n; ++i) {
      const int vi = sel_idx[i];
      const float xi = sel_val[i];
      int j = i - 1;
      while (j >= 0 && sel_idx[j] > vi) {
        sel_idx[j + 1] = sel_idx[j];
        sel_val[j + 1] = sel_val[j];
        --j;
      }
      sel_idx[j + 1] = vi;
      sel_val[j + 1] = xi;
    }
    const int e = a.row_exp[t];
    int32_t* oi = a.cand_idx + (size_t)t * kTopKMax;
    float* ov = a.cand_val + (size_t)t * kTopKMax;
    for (int j = 0; j < kTopKMax; ++j) {
      oi[j] = j < n ? sel_idx[j] : -1;
      ov[j] = j < n ? __builtin_ldexpf(sel_val[j], -e) : -__builtin_inff();
    }
  }
}

// Target weights of row t's candidates, exp((l - max l) / temperature), and
// their sum in ascending candidate order.
__device__ __forceinline__ float row_weights(const SampleArgs& a, int t, float (&w)[kTopKMax]) {
  const int32_t* ci = a.cand_idx + (size_t)t * kTopKMax;
  const float* cv = a.cand_val + (size_t)t * kTopKMax;
  float m = -__builtin_inff();
  for (int j = 0; j < kTopKMax; ++j)
    if (ci[j] >= 0 && cv[j] > m) m = cv[j];
  float tot = 0.0f;
  for (int j = 0; j < kTopKMax; ++j) {
    w[j] = (ci[j] >= 0 && m > -__builtin_inff()) ? expf((cv[j] - m) / a.temperature) : 0.0f;
    tot += w[j];
  }
  return tot;
}

// The candidate u picks by inverse CDF over the weights in ascending
// candidate (vocabulary) order, candidate `skip` left out.
__device__ __forceinline__ int pick(const float (&w)[kTopKMax], int skip, float u) {
  float tot = 0.0f;
  for (int j = 0; j < kTopKMax; ++j)
    if (j != skip) tot += w[j];
  const float x = u * tot;
  float c = 0.0f;
  int last = -1;
  for (int j = 0; j < kTopKMax; ++j) {
    if (j == skip || w[j] == 0.0f) continue;
    c += w[j];
    last = j;
    if (c > x) return j;
  }
  return last;  // past the end by rounding: the last candidate with weight
}

// One thread per group: accept drafts while u_acc < p(draft); at the first
// rejection emit a sample of p without the draft; after the last draft emit
// a sample of p (the bonus token).  A row without candidates rejects its
// draft and emits -1.
__global__ __launch_bounds__(64) void k_sample_verify(SampleArgs a) {
  const int g = threadIdx.x;
  if (g >= a.G) return;
  const int r = a.gs[g], n = a.gs[g + 1] - a.gs[g];
  int acc = 0;
  for (int i = 0; i < n; ++i) a.tokens[r + i] = -1;
  float w[kTopKMax];
  while (true) {
    const int t = r + acc;
    const float tot = row_weights(a, t, w);
    if (tot == 0.0f) break;
    const int32_t* ci = a.cand_idx + (size_t)t * kTopKMax;
    int skip = -1;
    if (acc < n - 1) {
      const int d = a.drafts[r - g + acc];
      for (int j = 0; j < kTopKMax; ++j)
        if (d >= 0 && ci[j] == d) skip = j;
      const float pd = skip >= 0 ? w[skip] / tot : 0.0f;
      if (a.u_acc[t] < pd) {
        a.tokens[t] = d;
        ++acc;
        continue;
      }
    }
    const int j = pick(w, skip, a.u_samp[t]);
    a.tokens[t] = j >= 0 ? ci[j] : -1;
    break;
  }
  a.n_acc[g] = acc;
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_topk, dim3(a.T), dim3(kTopKThreads), 0, st, a);
  hipLaunchKernelGGL(k_sample_verify, dim3(1), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace mk
