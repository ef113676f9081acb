// mk_gemv.hip — activation quantizer and the T-row Q4_K-style GEMV (both
// inner-product engines) with its split-K reduction fused: the last block of
// a tile to finish sums the tile's block partials in split order and either
// stores y or, for the gate/up pair of the FFN, applies SiLU(g) * u and
// quantizes the result as the down projection's activation rows.
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
                                                  int32_t* __restrict__ gsum, float2* __restrict__ ssg,
                                                  unsigned* __restrict__ zero, int nzero) {
  const int t = blockIdx.y;
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < nzero; i += 256) zero[i] = 0u;  // counters of the GEMV launches that follow
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
                           unsigned* zero, int nzero, hipStream_t st) {
  const int ng = K / 32;
  dim3 grid((ng + 7) / 8, T);
  hipLaunchKernelGGL(k_quantize, grid, dim3(256), 0, st, x, T, K, a8, s, gsum, ssg, zero, nzero);
  return hipGetLastError();
}

// ---------------------------------------------------------------- GEMV
struct GemvArgs {
  const uint8_t* W[2];
  int nsb, per_wg;
  QAct act;
  float* partial;  // [nmat][ksplit][T][ntiles*64]
  int ksplit, npad;
  unsigned* tickets;  // [ntiles] arrivals per tile; zero at launch
  int epi, n_out;
  float* y;      // kEpiStore: [T][n_out]; kEpiSiluQ8: h [T][n_out] fp32 or null
  int8_t* h8;    // kEpiSiluQ8: a8 [T][n_out]
  float2* hssg;  // kEpiSiluQ8: [n_out/32][kTPad]
};

// The block's 4 wave sums (red[w][t][r], rows of stride rs) are added in wave
// order and stored as its partial; the block that completes the tile's
// count of nmat * ksplit arrivals then runs the tile epilogue.
__device__ __forceinline__ void gemv_tile_end(const GemvArgs& a, const float* red, int rs, int T) {
  __shared__ int last;
  const int tile = blockIdx.x, ks = blockIdx.y, mat = blockIdx.z;
  for (int idx = threadIdx.x; idx < T * 64; idx += 256) {
    const int t = idx >> 6, r = idx & 63;
    const float v = ((red[(0 * rs + t) * 64 + r] + red[(1 * rs + t) * 64 + r]) + red[(2 * rs + t) * 64 + r]) +
                    red[(3 * rs + t) * 64 + r];
    st_coh(a.partial + (((size_t)mat * a.ksplit + ks) * T + t) * a.npad + (size_t)tile * 64 + r, v);
  }
  stores_done();  // every wave's partial stores are in memory before the ticket
  __syncthreads();
  if (threadIdx.x == 0) last = ticket_add(a.tickets + tile) == (unsigned)(a.ksplit * (int)gridDim.z) - 1u;
  __syncthreads();
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, o = tile * 64 + lane;
  const size_t mstride = (size_t)a.ksplit * T * a.npad;
  for (int t = w; t < T; t += 4) {
    float g = 0.0f, u = 0.0f;
    for (int k = 0; k < a.ksplit; ++k) g += ld_coh(a.partial + ((size_t)k * T + t) * a.npad + o);
    if (a.epi == kEpiStore) {
      if (o < a.n_out) a.y[(size_t)t * a.n_out + o] = g;
      continue;
    }
    for (int k = 0; k < a.ksplit; ++k) u += ld_coh(a.partial + mstride + ((size_t)k * T + t) * a.npad + o);
    const float h = g * u / (1.0f + expf(-g));
    if (a.y) a.y[(size_t)t * a.n_out + o] = h;
    // rows o of the tile are 2 activation groups of 32 (n_out % 256 == 0)
    const Q8 q = quant_group32(h);
    a.h8[(size_t)t * a.n_out + o] = (int8_t)q.a8;
    if ((lane & 31) == 0) a.hssg[(size_t)(o >> 5) * kTPad + t] = make_float2(q.s, q.s * (float)q.gsum);
  }
  if (a.epi == kEpiSiluQ8)
    for (int i = threadIdx.x; i < 2 * (kTPad - T); i += 256)  // padded rows t >= T of the tile's 2 groups
      a.hssg[(size_t)(2 * tile + i / (kTPad - T)) * kTPad + T + i % (kTPad - T)] = make_float2(0.0f, 0.0f);
}

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
  gemv_tile_end(a, &red[0][0][0], T, T);
}

// Block = 4 waves on one 64-row tile, as above; the block's activation rows
// (superblocks [lo, hi)) are staged in LDS while each wave's first unit
// loads.  A unit is loaded with 9 16-B loads per lane (lane = row, as for
// dot4) and the next unit's loads are in flight while the current one is
// transposed through the wave's LDS area into the matrix-core operand
// layout and multiplied.
__global__ __launch_bounds__(256) void k_gemv_mfma(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t act_lds[];  // per_wg x kActSbBytes
  // per wave: one unit in its global byte layout; after the loop, the wave sums
  __shared__ __attribute__((aligned(16))) uint8_t wl[4][kUnitBytes];
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
  uint8_t* mine = &wl[w][0];
  Unit ua, ub;  // ping-pong buffers: the next unit's loads are issued before this unit's arithmetic
  if (b0 < b1) load_unit(tileW + (size_t)b0 * kUnitBytes, lane, ua);
  stage_act(a.act, lo, n, act_lds);
  __syncthreads();
  for (int b = b0; b < b1; b += 2) {
    if (b + 1 < b1) load_unit(tileW + (size_t)(b + 1) * kUnitBytes, lane, ub);
    {
      UnitM x;
      transpose_unit(ua, mine, nl, kq, lane, x);
      mfma_unit(x, act_lds + (b - lo) * kActSbBytes, nl, kq, acc);
    }
    if (b + 1 >= b1) break;
    if (b + 2 < b1) load_unit(tileW + (size_t)(b + 2) * kUnitBytes, lane, ua);
    {
      UnitM x;
      transpose_unit(ub, mine, nl, kq, lane, x);
      mfma_unit(x, act_lds + (b + 1 - lo) * kActSbBytes, nl, kq, acc);
    }
  }
  __syncthreads();  // every wave is done with its unit area before it holds the sums
  float(*red)[kTPad][64] = (float(*)[kTPad][64])&wl[0][0];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w][4 * kq + i][16 * g + nl] = acc[g][i];
  __syncthreads();
  gemv_tile_end(a, &red[0][0][0], kTPad, a.act.T);
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
  if (spw > 2) spw = 2;  // at most 8 superblocks per block: its staged activation rows fit 40 KB of LDS
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
                       const GemvEpi& epi, hipStream_t st) {
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
  a.tickets = epi.tickets;
  a.epi = epi.kind;
  a.n_out = epi.n_out;
  a.y = epi.y;
  a.h8 = epi.h8;
  a.hssg = (float2*)epi.hssg;
  dim3 grid(p.ntiles, p.ksplit, p.nmat);
  if (path == 2) {
    hipLaunchKernelGGL(k_gemv_mfma, grid, dim3(256), (size_t)p.per_wg * kActSbBytes, st, a);
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

}  // namespace mk
