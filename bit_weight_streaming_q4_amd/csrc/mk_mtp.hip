// mk_mtp.hip — the on-device MTP draft loop (richland.au single-stream
// article, "What shipped": after verification, MTP catch-up rows for the
// accepted tokens, then n_draft MTP draft steps, drafting restricted to the
// 32,768 most frequent tokens; the 4-agent article, "Why it matters": each
// agent's drafts ride in the same rows).  Every pass runs the synthetic draft
// head on all of its rows with one weight read (the T-row GEMV and FFN
// launches); the token that feeds the next pass and the row that continues
// each group's chain are read from device memory, so no step of the loop
// returns to the host.
//
// One pass over rows (token, hidden):
//   z  = [RMSNorm(f32 E[token]) ; RMSNorm(hidden)]     (k_mtp_in)
//   u  = fc . q8(z)                                      (T-row GEMV)
//   x' = u + FFN(RMSNorm(u))                             (k_rms_rows, FFN, k_mtp_add)
//   per group: the row that continues the chain -> RMSNorm -> argmax over the
//   draft-vocabulary prefix of the tied lm_head          (k_mtp_sel, lm_head)
#include "mk_device.h"
#include "mk_internal.h"

namespace mk {

constexpr int kMtpThreads = 256;
constexpr float kMtpEps = 1e-6f;

// Sum over the block (256 threads); every thread gets the same value.
__device__ __forceinline__ float block_sum256(float v, float* red) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Row i of the pass input z [rows][2H].  Pass 0 (the catch-up pass): row i
// of the step with its emitted token; rows past their group's accept length
// are not catch-up rows and get zeros.  Pass k > 0: row g continues group g's
// chain with draft k - 1 and the x' of the row that produced it.
__global__ __launch_bounds__(kMtpThreads) void k_mtp_in(MtpArgs a, int pass) {
  __shared__ float red[4];
  const int i = blockIdx.x, tid = threadIdx.x, H = a.H;
  int tok;
  const float* h;
  bool live = true;
  if (pass == 0) {
    int g = 0;
    while (g + 1 < a.G && i >= a.gs[g + 1]) ++g;
    const int n = a.n_acc[g];
    live = n >= 0 && n < a.gs[g + 1] - a.gs[g] && i - a.gs[g] <= n;
    tok = a.tokens[i];
    h = a.hidden + (size_t)i * H;
  } else {
    tok = a.drafts[(size_t)(pass - 1) * a.G + i];
    h = a.prev + (size_t)i * H;
  }
  float* z = a.z + (size_t)i * 2 * H;
  const bool emb = live && tok >= 0 && tok < a.V;
  const uint16_t* e = a.embed + (size_t)(emb ? tok : 0) * H;
  float se = 0.0f, sh = 0.0f;
  for (int j = tid; j < H; j += kMtpThreads) {
    const float ev = emb ? f16_bits_to_f32(e[j]) : 0.0f;
    const float hv = live ? h[j] : 0.0f;
    se = __builtin_fmaf(ev, ev, se);
    sh = __builtin_fmaf(hv, hv, sh);
  }
  se = block_sum256(se, red);
  sh = block_sum256(sh, red);
  const float re = 1.0f / __builtin_sqrtf(se / (float)H + kMtpEps), rh = 1.0f / __builtin_sqrtf(sh / (float)H + kMtpEps);
  for (int j = tid; j < H; j += kMtpThreads) {
    z[j] = emb ? f16_bits_to_f32(e[j]) * re : 0.0f;
    z[H + j] = live ? h[j] * rh : 0.0f;
  }
}

// out[i] = RMSNorm(in[i]) (unit gain), one block per row.
__global__ __launch_bounds__(kMtpThreads) void k_rms_rows(const float* __restrict__ in, float* __restrict__ out, int H) {
  __shared__ float red[4];
  const float* x = in + (size_t)blockIdx.x * H;
  float s = 0.0f;
  for (int j = threadIdx.x; j < H; j += kMtpThreads) s = __builtin_fmaf(x[j], x[j], s);
  s = block_sum256(s, red);
  const float r = 1.0f / __builtin_sqrtf(s / (float)H + kMtpEps);
  for (int j = threadIdx.x; j < H; j += kMtpThreads) out[(size_t)blockIdx.x * H + j] = x[j] * r;
}

// x' = u + y for every row of the pass; the trace (optional) receives it.
__global__ __launch_bounds__(kMtpThreads) void k_mtp_add(MtpArgs a, int rows, int trace_row0) {
  const size_t n = (size_t)rows * a.H;
  for (size_t j = (size_t)blockIdx.x * kMtpThreads + threadIdx.x; j < n; j += (size_t)gridDim.x * kMtpThreads) {
    const float v = a.u[j] + a.y[j];
    a.xp[j] = v;
    if (a.trace) a.trace[(size_t)trace_row0 * a.H + j] = v;
  }
}

// Per group g: the row that continues the chain (pass 0: row gs[g] + n_acc[g];
// later passes: row g) becomes prev[g], and hid[g] = RMSNorm of it feeds the
// lm_head.  A group whose accept length is outside 0..rows-1 is dead: its
// hid rows are NaN, so every draft of it is -1 (NaN never wins the argmax).
__global__ __launch_bounds__(kMtpThreads) void k_mtp_sel(MtpArgs a, int pass) {
  __shared__ float red[4];
  const int g = blockIdx.x, H = a.H;
  int row = g;
  if (pass == 0) {
    const int n = a.n_acc[g];
    const bool ok = n >= 0 && n < a.gs[g + 1] - a.gs[g];
    if (threadIdx.x == 0) a.dead[g] = ok ? 0 : 1;
    row = a.gs[g] + (ok ? n : 0);
  }
  __syncthreads();
  const bool dead = pass == 0 ? !(a.n_acc[g] >= 0 && a.n_acc[g] < a.gs[g + 1] - a.gs[g]) : a.dead[g] != 0;
  const float* x = a.xp + (size_t)row * H;
  float s = 0.0f;
  for (int j = threadIdx.x; j < H; j += kMtpThreads) s = __builtin_fmaf(x[j], x[j], s);
  s = block_sum256(s, red);
  const float r = 1.0f / __builtin_sqrtf(s / (float)H + kMtpEps);
  for (int j = threadIdx.x; j < H; j += kMtpThreads) {
    a.prev[(size_t)g * H + j] = x[j];
    a.hid[(size_t)g * H + j] = dead ? __builtin_nanf("") : x[j] * r;
  }
}

hipError_t launch_mtp_in(const MtpArgs& a, int pass, int rows, hipStream_t st) {
  hipLaunchKernelGGL(k_mtp_in, dim3(rows), dim3(kMtpThreads), 0, st, a, pass);
  return hipGetLastError();
}

hipError_t launch_rms_rows(const float* in, float* out, int rows, int H, hipStream_t st) {
  hipLaunchKernelGGL(k_rms_rows, dim3(rows), dim3(kMtpThreads), 0, st, in, out, H);
  return hipGetLastError();
}

hipError_t launch_mtp_out(const MtpArgs& a, int pass, int rows, int trace_row0, hipStream_t st) {
  const int blocks = (int)(((size_t)rows * a.H + kMtpThreads - 1) / kMtpThreads);
  hipLaunchKernelGGL(k_mtp_add, dim3(blocks), dim3(kMtpThreads), 0, st, a, rows, trace_row0);
  hipLaunchKernelGGL(k_mtp_sel, dim3(a.G), dim3(kMtpThreads), 0, st, a, pass);
  return hipGetLastError();
}

}  // namespace mk
