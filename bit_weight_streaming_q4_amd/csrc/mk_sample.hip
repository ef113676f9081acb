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

constexpr int kTopKThreads = 256;
constexpr int kTopKChunk = 8192;  // logits per first-level block (staged in LDS)

// Inclusive prefix sum of v over the block's 256 threads in thread order.
__device__ __forceinline__ unsigned block_scan256(unsigned v, unsigned* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  unsigned off = 0;
  for (int i = 0; i < w; ++i) off += wsum[i];
  __syncthreads();
  return v + off;
}

// The bin holding the rem-th element, counting bins from the top (DESC) or
// from the bottom: its digit, how many of it are still needed, and its
// count, into sh[1..3].  One bin per thread; the thread whose running count
// first reaches rem writes.
template <bool DESC>
__device__ __forceinline__ void find_bin(const unsigned* hist, unsigned rem, unsigned* sh, unsigned* wsum) {
  const int d = DESC ? 255 - (int)threadIdx.x : (int)threadIdx.x;
  const unsigned c = hist[d];
  const unsigned incl = block_scan256(c, wsum);
  if (incl >= rem && incl - c < rem) {
    sh[1] = (unsigned)d;
    sh[2] = rem - (incl - c);
    sh[3] = c;
  }
  __syncthreads();
}

// The k largest of n values val[i] with identities id[i] (both in LDS), NaN
// never counted, ties broken towards the lower identity: written to
// sel_id / sel_val (LDS, unordered); returns how many (min(k, non-NaN)).
// The k-th largest key comes from four 8-bit radix passes (MSB first); when
// several values equal it, the lowest identities are found by four more
// passes over those identities.  Every choice comes from exact counts, so
// the result does not depend on timing.  All threads of the block call it.
__device__ int block_topk(const float* val, const int* id, int n, int k, int* sel_id, float* sel_val,
                          unsigned* hist, unsigned* sh) {
  const int tid = threadIdx.x;
  // sh[0]: non-NaN count, [1]: digit, [2]: remaining, [3]: ties, [4]: selected,
  // [5]: smallest key, [6]: largest key, [8..11]: scan
  static_assert(kTopKThreads == 256, "one histogram bin per thread");
  if (tid == 0) {
    sh[0] = 0;
    sh[4] = 0;
    sh[5] = 0xFFFFFFFFu;
    sh[6] = 0;
  }
  __syncthreads();
  unsigned nn = 0, kmin = 0xFFFFFFFFu, kmax = 0;
  for (int i = tid; i < n; i += kTopKThreads) {
    if (val[i] != val[i]) continue;
    const uint32_t key = order_key(val[i]);
    ++nn;
    kmin = key < kmin ? key : kmin;
    kmax = key > kmax ? key : kmax;
  }
  if (nn) {
    atomicAdd(&sh[0], nn);
    atomicMin(&sh[5], kmin);
    atomicMax(&sh[6], kmax);
  }
  __syncthreads();
  const unsigned keff = sh[0] < (unsigned)k ? sh[0] : (unsigned)k;
  if (keff == 0) return 0;
  // Radix select of the keff-th largest key on d = key - (smallest key),
  // 8 bits at a time from the top bit of the range down: the first digit
  // already spreads the values over the bins.
  const uint32_t base = sh[5];
  const uint32_t range = sh[6] - base;
  int hi = range ? 32 - __builtin_clz(range) : 0;  // bits of d still to decide
  uint64_t P = 0;                                  // the decided high bits of d
  unsigned rem = keff, n_eq = sh[0];
  while (hi > 0) {
    const int lo = hi > 8 ? hi - 8 : 0, width = hi - lo;
    const uint32_t wmask = (1u << width) - 1u;
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopKThreads) {
      if (val[i] != val[i]) continue;
      const uint64_t d = (uint64_t)(order_key(val[i]) - base);
      if ((d >> hi) == P) atomicAdd(&hist[(uint32_t)(d >> lo) & wmask], 1u);
    }
    __syncthreads();
    find_bin<true>(hist, rem, sh, sh + 8);
    P = (P << width) | sh[1];
    rem = sh[2];
    n_eq = sh[3];
    hi = lo;
    __syncthreads();
  }
  const uint32_t kth = base + (uint32_t)P;
  uint32_t id_max = 0xFFFFFFFFu;  // every tie qualifies when all are taken
  if (n_eq > rem) {
    uint32_t ip = 0, imask = 0;
    unsigned irem = rem;
    for (int p = 0; p < 4; ++p) {
      const int shift = 24 - 8 * p;
      hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kTopKThreads)
        if (val[i] == val[i] && order_key(val[i]) == kth && ((uint32_t)id[i] & imask) == ip)
          atomicAdd(&hist[((uint32_t)id[i] >> shift) & 255u], 1u);
      __syncthreads();
      find_bin<false>(hist, irem, sh, sh + 8);
      ip |= sh[1] << shift;
      imask |= 0xFFu << shift;
      irem = sh[2];
      __syncthreads();
    }
    id_max = ip;  // the rem-th lowest identity among the ties
  }
  for (int i = tid; i < n; i += kTopKThreads) {
    if (val[i] != val[i]) continue;
    const uint32_t key = order_key(val[i]);
    if (key > kth || (key == kth && (uint32_t)id[i] <= id_max)) {
      const unsigned slot = atomicAdd(&sh[4], 1u);
      if (slot < (unsigned)kTopKMax) {
        sel_id[slot] = id[i];
        sel_val[slot] = val[i];
      }
    }
  }
  __syncthreads();
  return (int)(sh[4] < keff ? sh[4] : keff);
}

// (va, ia) ranks above (vb, ib): the larger value, then the lower identity.
__device__ __forceinline__ bool beats(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

constexpr int kCandCap = 1024;  // candidates the threshold pass may collect

struct TopkScratch {
  float tm_val[kTopKThreads];  // per-thread maxima
  int tm_id[kTopKThreads];
  float cand_val[kCandCap];
  int cand_id[kCandCap];
  unsigned hist[256];
  unsigned sh[16];
};

// The same selection as block_topk, usually much cheaper: the k-th largest
// of the 256 per-thread maxima is a lower bound on the k-th largest value
// (the top k maxima are k distinct values at least that large), so every
// value of the top k is at least it.  One pass collects the values at least
// that large (a few more than k unless the values cluster), and each one's
// rank among them (how many others rank above it) places the k best
// exactly.  If more than kCandCap values qualify, block_topk runs instead.
// sel_id / sel_val receive the top k in rank order.
__device__ int block_topk_fast(const float* val, const int* id, int n, int k, int* sel_id, float* sel_val,
                               TopkScratch& w) {
  const int tid = threadIdx.x;
  float bm = 0.0f;
  int bi = -1;
#pragma unroll 8
  for (int i = tid; i < n; i += kTopKThreads) {
    const float x = val[i];
    if (x == x && (bi < 0 || beats(x, id[i], bm, bi))) {
      bm = x;
      bi = id[i];
    }
  }
  w.tm_val[tid] = bm;
  w.tm_id[tid] = bi;
  if (tid == 0) {
    w.sh[0] = 0;  // valid thread maxima
    w.sh[1] = 0;  // collected candidates
    w.sh[2] = 0;  // threshold found
  }
  __syncthreads();
  if (bi >= 0) {
    atomicAdd(&w.sh[0], 1u);
    int r = 0;
#pragma unroll 32
    for (int j = 0; j < kTopKThreads; ++j) r += w.tm_id[j] >= 0 && beats(w.tm_val[j], w.tm_id[j], bm, bi);
    if (r == k - 1) {  // exactly one thread when at least k threads hold a value
      w.sh[2] = 1;
      w.sh[3] = __builtin_bit_cast(unsigned, bm);
    }
  }
  __syncthreads();
  // fewer than k threads hold a value: every value qualifies
  const float theta = w.sh[2] ? __builtin_bit_cast(float, w.sh[3]) : -__builtin_inff();
#pragma unroll 8
  for (int i = tid; i < n; i += kTopKThreads) {
    const float x = val[i];
    if (x == x && x >= theta) {
      const unsigned slot = atomicAdd(&w.sh[1], 1u);
      if (slot < (unsigned)kCandCap) {
        w.cand_val[slot] = x;
        w.cand_id[slot] = id[i];
      }
    }
  }
  __syncthreads();
  const int m = (int)w.sh[1];
  if (m > kCandCap) return block_topk(val, id, n, k, sel_id, sel_val, w.hist, w.sh);
  for (int c = tid; c < m; c += kTopKThreads) {
    const float vc = w.cand_val[c];
    const int ic = w.cand_id[c];
    int r = 0;
#pragma unroll 16
    for (int d = 0; d < m; ++d) r += beats(w.cand_val[d], w.cand_id[d], vc, ic);
    if (r < k) {
      sel_id[r] = ic;
      sel_val[r] = vc;
    }
  }
  __syncthreads();
  return m < k ? m : k;
}

// First level: block (c, t) stages logits [c * kTopKChunk, ...) of row t in
// LDS and writes that chunk's top-k candidates (identity = vocabulary index;
// -1 / NaN past the chunk's count) to part [t][c][32].  The row's top-k is
// within the union of its chunks' top-k (an element that loses inside its
// chunk loses to k elements that also outrank it in the row).
__global__ __launch_bounds__(kTopKThreads) void k_topk_chunk(SampleArgs a, int32_t* part_id, float* part_val,
                                                             int nchunk) {
  __shared__ float val[kTopKChunk];
  __shared__ int id[kTopKChunk];
  __shared__ TopkScratch w;
  __shared__ int sel_id[kTopKMax];
  __shared__ float sel_val[kTopKMax];
  const int c = blockIdx.x, t = blockIdx.y;
  const int v0 = c * kTopKChunk, n = a.V - v0 < kTopKChunk ? a.V - v0 : kTopKChunk;
  const float* row = a.logits + (size_t)t * a.V + v0;
  // all of a thread's loads in flight before any is written to LDS
  constexpr int kPer = kTopKChunk / kTopKThreads;
  float v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = j * kTopKThreads + threadIdx.x;
    v[j] = i < n ? row[i] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = j * kTopKThreads + threadIdx.x;
    if (i < n) {
      val[i] = v[j];
      id[i] = v0 + i;
    }
  }
  __syncthreads();
  const int m = block_topk_fast(val, id, n, a.k, sel_id, sel_val, w);
  if (threadIdx.x < kTopKMax) {
    const size_t o = ((size_t)t * nchunk + c) * kTopKMax + threadIdx.x;
    part_id[o] = (int)threadIdx.x < m ? sel_id[threadIdx.x] : -1;
    part_val[o] = (int)threadIdx.x < m ? sel_val[threadIdx.x] : __builtin_nanf("");
  }
}

// Second level: one block per row selects the top-k among its chunks'
// candidates and writes them in ascending vocabulary order, scaled back by
// 2^-row_exp[t].
__global__ __launch_bounds__(kTopKThreads) void k_topk_merge(SampleArgs a, const int32_t* part_id,
                                                             const float* part_val, int nchunk) {
  extern __shared__ uint8_t smem[];
  __shared__ TopkScratch w;
  __shared__ int sel_id[kTopKMax];
  __shared__ float sel_val[kTopKMax];
  const int t = blockIdx.x, n = nchunk * kTopKMax;
  float* val = (float*)smem;
  int* id = (int*)(smem + (size_t)n * 4);
  for (int i0 = 0; i0 < n; i0 += 8 * kTopKThreads) {  // eight loads of each kind in flight per thread
    float pv[8];
    int pi[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * kTopKThreads + threadIdx.x;
      pv[j] = i < n ? part_val[(size_t)t * n + i] : 0.0f;
      pi[j] = i < n ? part_id[(size_t)t * n + i] : -1;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j * kTopKThreads + threadIdx.x;
      if (i < n) {
        val[i] = pv[j];
        id[i] = pi[j];
      }
    }
  }
  __syncthreads();
  const int m = block_topk(val, id, n, a.k, sel_id, sel_val, w.hist, w.sh);
  // ascending vocabulary order: candidate j goes to its rank among the m
  // (the identities are distinct)
  const int j = threadIdx.x, e = a.row_exp[t];
  int32_t* oi = a.cand_idx + (size_t)t * kTopKMax;
  float* ov = a.cand_val + (size_t)t * kTopKMax;
  if (j < m) {
    int rank = 0;
    for (int i = 0; i < m; ++i) rank += sel_id[i] < sel_id[j];
    oi[rank] = sel_id[j];
    ov[rank] = __builtin_ldexpf(sel_val[j], -e);
  } else if (j < kTopKMax) {
    oi[j] = -1;
    ov[j] = -__builtin_inff();
  }
}

int topk_chunks(int V) { return (V + kTopKChunk - 1) / kTopKChunk; }

// Sum over the wave (every lane gets the same value).
__device__ __forceinline__ float wave_sum_f(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One wave per group, lane j = candidate j of the current row: accept drafts
// while u_acc < p(draft); at the first rejection emit a sample of p without
// the draft; after the last draft emit a sample of p (the bonus token).  The
// weights are exp((l - max l) / temperature); a sample is the first
// candidate, in ascending vocabulary order, whose running weight exceeds
// u * total.  A row without candidates rejects its draft and emits -1.
__global__ __launch_bounds__(64) void k_sample_verify(SampleArgs a) {
  const int g = blockIdx.x, j = threadIdx.x;
  const int r = a.gs[g], n = a.gs[g + 1] - a.gs[g];
  for (int i = j; i < n; i += 64) a.tokens[r + i] = -1;
  int acc = 0;
  while (true) {
    const int t = r + acc;
    const int ci = j < kTopKMax ? a.cand_idx[(size_t)t * kTopKMax + j] : -1;
    const float cv = j < kTopKMax ? a.cand_val[(size_t)t * kTopKMax + j] : 0.0f;
    const bool live = ci >= 0;
    float m = live ? cv : -__builtin_inff();
    for (int o = 32; o >= 1; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, 64));
    const float w = (live && m > -__builtin_inff()) ? expf((cv - m) / a.temperature) : 0.0f;
    const float tot = wave_sum_f(w);
    if (tot == 0.0f) break;
    int skip = -1;
    if (acc < n - 1) {
      const int d = a.drafts[r - g + acc];
      const uint64_t hit = __ballot(live && d >= 0 && ci == d);
      if (hit) skip = __builtin_ctzll(hit);
      const float pd = skip >= 0 ? __shfl(w, skip, 64) / tot : 0.0f;
      if (a.u_acc[t] < pd) {
        if (j == 0) a.tokens[t] = d;
        ++acc;
        continue;
      }
    }
    // inverse CDF without the rejected draft
    const float wk = j == skip ? 0.0f : w;
    float c = wk;
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(c, o, 64);
      if (j >= o) c += y;
    }
    const float x = a.u_samp[t] * __shfl(c, 63, 64);
    const uint64_t over = __ballot(wk > 0.0f && c > x);
    const uint64_t any = __ballot(wk > 0.0f);
    const int pick = over ? __builtin_ctzll(over) : (any ? 63 - __builtin_clzll(any) : -1);
    const int tok = pick >= 0 ? __shfl(ci, pick, 64) : -1;
    if (j == 0) a.tokens[t] = tok;
    break;
  }
  if (j == 0) a.n_acc[g] = acc;
}

size_t sample_part_bytes(int V, int T) { return (size_t)T * topk_chunks(V) * kTopKMax * 8; }

hipError_t launch_sample(const SampleArgs& a, void* part, hipStream_t st) {
  const int nchunk = topk_chunks(a.V);
  int32_t* part_id = (int32_t*)part;
  float* part_val = (float*)((uint8_t*)part + (size_t)a.T * nchunk * kTopKMax * 4);
  hipLaunchKernelGGL(k_topk_chunk, dim3(nchunk, a.T), dim3(kTopKThreads), 0, st, a, part_id, part_val, nchunk);
  hipLaunchKernelGGL(k_topk_merge, dim3(a.T), dim3(kTopKThreads), (size_t)nchunk * kTopKMax * 8, st, a, part_id,
                     part_val, nchunk);
  hipLaunchKernelGGL(k_sample_verify, dim3(a.G), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace mk
