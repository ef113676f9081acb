// mk_gemv.hip — activation quantizer and the T-row Q4_K-style GEMV (both
// inner-product engines), with the split-K reduction and the SiLU epilogue.
//
// The GEMV streams every weight unit from HBM exactly once per call and
// multiplies it against all T rows while it is in registers (pages:
// richland.au single-stream article, "What shipped" — shared activations so
// T rows cost about the memory time of one; 4-agent article, "Why it
// matters" — each loaded weight is multiplied against all 12 rows).
#include "mk_device.h"
#include "mk_internal.h"

namespace mk {

// ---------------------------------------------------------------- quantizer
// One wave per two 32-element groups of one row; block = 4 waves.
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ x, int T, int K,
                                                  int8_t* __restrict__ a8, float* __restrict__ s,
                                                  int32_t* __restrict__ gsum, float2* __restrict__ ssg) {
  const int t = blockIdx.y;
  const int ng = K / 32;
  const int g = blockIdx.x * 8 + (threadIdx.x >> 5);
  const int e = threadIdx.x & 31;
  const bool valid = g < ng;
  const float xv = valid ? x[(size_t)t * K + (size_t)g * 32 + e] : 0.0f;
  const Q8 q = quant_group32(xv);
  if (!valid) return;
  if (a8) a8[(size_t)t * K + (size_t)g * 32 + e] = (int8_t)q.a8;
  if (e == 0) {
    if (s) s[(size_t)t * ng + g] = q.s;
    if (gsum) gsum[(size_t)t * ng + g] = q.gsum;
    if (ssg) {
      ssg[(size_t)g * kTPad + t] = make_float2(q.s, q.s * (float)q.gsum);
      if (t == 0)
        for (int tt = T; tt < kTPad; ++tt) ssg[(size_t)g * kTPad + tt] = make_float2(0.0f, 0.0f);
    }
  }
}

hipError_t launch_quantize(const float* x, int T, int K, int8_t* a8, float* s, int32_t* gsum, float2* ssg,
                           hipStream_t st) {
  const int ng = K / 32;
  dim3 grid((ng + 7) / 8, T);
  hipLaunchKernelGGL(k_quantize, grid, dim3(256), 0, st, x, T, K, a8, s, gsum, ssg);
  return hipGetLastError();
}

// ---------------------------------------------------------------- GEMV
struct GemvArgs {
  const uint8_t* W[2];
  int nsb, per_wg;
  QAct act;
  float* partial;  // [nmat][ksplit][T][ntiles*64]
  int ksplit, npad;
};

// Block = 4 waves on one 64-row tile; the block's superblock range is split
// into 4 contiguous parts, one per wave; the 4 partial sums are added in wave
// order through LDS (fixed order, so the result is reproducible).
template <int T>
__global__ __launch_bounds__(256) void k_gemv_dot4(GemvArgs a) {
  __shared__ float red[4][T][64];
  const int tile = blockIdx.x, ks = blockIdx.y, mat = blockIdx.z;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int lo = ks * a.per_wg, hi = min(a.nsb, lo + a.per_wg);
  const int n = max(hi - lo, 0);
  const int b0 = lo + (n * w) / 4, b1 = lo + (n * (w + 1)) / 4;
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;
  const uint8_t* tileW = a.W[mat] + (size_t)tile * a.nsb * kUnitBytes;
  dot4_range<T>(tileW, b0, b1, a.act, lane, acc);
#pragma unroll
  for (int t = 0; t < T; ++t) red[w][t][lane] = acc[t];
  __syncthreads();
  for (int idx = threadIdx.x; idx < T * 64; idx += 256) {
    const int t = idx >> 6, r = idx & 63;
    const float v = ((red[0][t][r] + red[1][t][r]) + red[2][t][r]) + red[3][t][r];
    a.partial[(((size_t)mat * a.ksplit + ks) * T + t) * a.npad + (size_t)tile * 64 + r] = v;
  }
}

__global__ __launch_bounds__(256) void k_gemv_mfma(GemvArgs a) {
  __shared__ float red[4][kTPad][64];
  const int tile = blockIdx.x, ks = blockIdx.y, mat = blockIdx.z;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int nl = lane & 15, kq = lane >> 4;
  const int lo = ks * a.per_wg, hi = min(a.nsb, lo + a.per_wg);
  const int n = max(hi - lo, 0);
  const int b0 = lo + (n * w) / 4, b1 = lo + (n * (w + 1)) / 4;
  float acc[4][4];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[g][i] = 0.0f;
  const uint8_t* tileW = a.W[mat] + (size_t)tile * a.nsb * kUnitBytes;
  mfma_range(tileW, b0, b1, a.act, lane, acc);
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w][4 * kq + i][16 * g + nl] = acc[g][i];
  __syncthreads();
  const int T = a.act.T;
  for (int idx = threadIdx.x; idx < T * 64; idx += 256) {
    const int t = idx >> 6, r = idx & 63;
    const float v = ((red[0][t][r] + red[1][t][r]) + red[2][t][r]) + red[3][t][r];
    a.partial[(((size_t)mat * a.ksplit + ks) * T + t) * a.npad + (size_t)tile * 64 + r] = v;
  }
}

GemvPlan plan_gemv(int T, int n_out, int n_in, int nmat, int cu_count) {
  GemvPlan p;
  p.ntiles = (n_out + 63) / 64;
  p.nsb = n_in / 256;
  p.nmat = nmat;
  const long units = (long)p.ntiles * p.nsb * nmat;
  const long target_waves = (long)(cu_count > 0 ? cu_count : 256) * 16;
  int spw = (int)((units + target_waves - 1) / target_waves);
  if (spw < 1) spw = 1;
  p.per_wg = 4 * spw;
  if (p.per_wg > p.nsb) p.per_wg = p.nsb;
  p.ksplit = (p.nsb + p.per_wg - 1) / p.per_wg;
  p.partial_elems = (size_t)nmat * p.ksplit * T * (size_t)p.ntiles * 64;
  return p;
}

template <int T>
static void launch_dot4_t(const GemvArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL(k_gemv_dot4<T>, grid, dim3(256), 0, st, a);
}

hipError_t launch_gemv(const uint8_t* const* W, const GemvPlan& p, const QActBuf& act, int path, float* partial,
                       hipStream_t st) {
  GemvArgs a;
  a.W[0] = W[0];
  a.W[1] = p.nmat > 1 ? W[1] : W[0];
  a.nsb = p.nsb;
  a.per_wg = p.per_wg;
  a.act.a8 = act.a8;
  a.act.ssg = (const float*)act.ssg;
  a.act.K = act.K;
  a.act.T = act.T;
  a.partial = partial;
  a.ksplit = p.ksplit;
  a.npad = p.ntiles * 64;
  dim3 grid(p.ntiles, p.ksplit, p.nmat);
  if (path == 2) {
    hipLaunchKernelGGL(k_gemv_mfma, grid, dim3(256), 0, st, a);
  } else {
    switch (act.T) {
      case 1: launch_dot4_t<1>(a, grid, st); break;
      case 2: launch_dot4_t<2>(a, grid, st); break;
      case 3: launch_dot4_t<3>(a, grid, st); break;
      case 4: launch_dot4_t<4>(a, grid, st); break;
      case 5: launch_dot4_t<5>(a, grid, st); break;
      case 6: launch_dot4_t<6>(a, grid, st); break;
      case 7: launch_dot4_t<7>(a, grid, st); break;
      case 8: launch_dot4_t<8>(a, grid, st); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- reductions
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ partial, int ksplit, int T, int npad,
                                                int n_out, float* __restrict__ y) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * n_out) return;
  const int t = idx / n_out, o = idx % n_out;
  float v = 0.0f;
  for (int ks = 0; ks < ksplit; ++ks) v += partial[((size_t)ks * T + t) * npad + o];
  y[(size_t)t * n_out + o] = v;
}

__global__ __launch_bounds__(256) void k_reduce_silu(const float* __restrict__ partial, int ksplit, int T,
                                                     int npad, int n_out, float* __restrict__ h) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * n_out) return;
  const int t = idx / n_out, o = idx % n_out;
  float g = 0.0f, u = 0.0f;
  const size_t mstride = (size_t)ksplit * T * npad;
  for (int ks = 0; ks < ksplit; ++ks) {
    g += partial[((size_t)ks * T + t) * npad + o];
    u += partial[mstride + ((size_t)ks * T + t) * npad + o];
  }
  h[(size_t)t * n_out + o] = g * u / (1.0f + expf(-g));
}

hipError_t launch_reduce(const float* partial, const GemvPlan& p, int T, int n_out, float* y, hipStream_t st) {
  const int n = T * n_out;
  hipLaunchKernelGGL(k_reduce, dim3((n + 255) / 256), dim3(256), 0, st, partial, p.ksplit, T, p.ntiles * 64,
                     n_out, y);
  return hipGetLastError();
}

hipError_t launch_reduce_silu(const float* partial, const GemvPlan& p, int T, int n_out, float* h,
                              hipStream_t st) {
  const int n = T * n_out;
  hipLaunchKernelGGL(k_reduce_silu, dim3((n + 255) / 256), dim3(256), 0, st, partial, p.ksplit, T,
                     p.ntiles * 64, n_out, h);
  return hipGetLastError();
}

}  // namespace mk
