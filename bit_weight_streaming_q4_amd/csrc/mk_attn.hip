// mk_attn.hip — full-attention decode of T query rows over an fp16 KV cache
// (richland.au, "Fusing the whole speculative-decoding cycle into one CUDA
// kernel", section "What shipped": the attention layers decode with split-K
// flash decoding over an fp16 KV cache, tensor-core products on K/V tiles).
//
// Work split: one wave owns one item = (agent g, KV head h, split s), the
// positions [s*chunk, min(L_g, (s+1)*chunk)) of that agent's cache, and all
// query columns that read KV head h: the agent's n_g rows x the Hq/Hkv query
// heads of the group (NQ <= 16*NB columns).  The four waves of a block take
// four adjacent splits of one head and merge them through LDS into one
// partial; a second launch merges the partials of each (row, query head)
// and applies the output gate.
//
// Per 64-position tile the wave computes the transposed scores
//   S^T[pos][col] = K[pos] . q[col]            (v_mfma_f32_16x16x32_f16)
// and accumulates
//   O^T[dim][col] += V^T[dim][pos] P^T[pos][col]
// so that every lane holds one query column in both products: the online
// softmax (running max, rescale) stays inside the lane and its three
// neighbours at distance 16, 32, 48.  The MFMA k index is permuted so that
// each lane's operands are 16 contiguous bytes: K rows are position-major
// (lane group j reads dims 32m + 8j .. +7 of its position in product m), and
// the V cache is dimension-major, so a lane reads 8 consecutive positions of
// one dimension.  Score block b (16 positions) maps its row r to position
// 32(b/2) + 8(r/4) + 4(b%2) + r%4, which puts positions 32hh + 8j .. +7 of
// half tile hh in lane group j: exactly the B operand the PV product needs.
//
// Precision: K and V are fp16 (exact in the products).  q * log2(e)/sqrt(d)
// and the probabilities p are split into fp16 hi + lo parts (split_f16), so
// both products carry about 22 bits; accumulation is fp32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mk.h"
#include "mk_attn.h"
#include "mk_internal.h"

namespace mk {
namespace {

using namespace attn;

constexpr int kWaves = 4;
constexpr int kMergeFloats = 34;  // per lane and column block: 32 outputs, max, sum

// Q8: the cache holds q8_0 blocks (32 int8 codes, one fp16 scale).  Each score
// product m covers exactly the 32-dim block m of a K row, and each P.V
// product exactly one 32-position block of a V row, so a product runs on the
// codes (exact in fp16) and its result is scaled per row in fp32.
// One column block fits two waves per SIMD (256 registers with the matrix
// accumulators); more column blocks run one wave per SIMD.
template <int NB, bool Q8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NB == 1 ? 2 : 1)))
void k_attn_split(const AttnArgs a) {
  // q slots [w][nb][m][hi/lo][lane] during the loop; afterwards the four
  // waves' results [w][nb][34][lane] for the merge.
  __shared__ float smem[kWaves * NB * kMergeFloats * 64];
  u4* qs = (u4*)smem;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // The item count is a multiple of 4 and the grid has one block per 4 items,
  // so no wave is idle; a block's waves take splits 4q .. 4q+3 of one head.
  // wave-uniform, so that everything derived from it (the item, its
  // positions, every tile test) stays in scalar registers and branches
  const int it = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + w);
  int g = 0;
  while (it >= a.item0[g + 1]) ++g;
  const int loc = it - a.item0[g], ns = a.nsplit[g];
  const int h = loc / ns, s = loc - h * ns;
  const int r0 = a.gs[g], ng = a.gs[g + 1] - r0, ctx = a.ctx[g], Lg = ctx + ng;
  const int p0 = s * a.chunk, p1 = min(Lg, p0 + a.chunk);
  const int gqa = a.gqa, NQ = ng * gqa;
  const int col = lane & 15, grp = lane >> 4;

  // Query columns: scaled, split into fp16 hi + lo, parked in this lane's own
  // LDS slots (read back every tile, so they need no registers meanwhile).
  int lim[NB];  // positions < lim[nb] are visible to this lane's column
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int c = nb * 16 + col;
    const bool valid = c < NQ;
    const int row = r0 + (valid ? c / gqa : 0), hq = h * gqa + (valid ? c % gqa : 0);
    lim[nb] = valid ? min(ctx + c / gqa + 1, p1) : 0;
    const float* qr = a.q + ((size_t)row * a.Hq + hq) * kD + 8 * grp;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float4 u0 = make_float4(0.f, 0.f, 0.f, 0.f), u1 = u0;
      if (valid) {
        u0 = *(const float4*)(qr + 32 * m);
        u1 = *(const float4*)(qr + 32 * m + 4);
      }
      const float x[8] = {u0.x * a.qscale, u0.y * a.qscale, u0.z * a.qscale, u0.w * a.qscale,
                          u1.x * a.qscale, u1.y * a.qscale, u1.z * a.qscale, u1.w * a.qscale};
      u4 hi, lo;
      split_f16(x, hi, lo);
      qs[(((w * NB + nb) * 4 + m) * 2 + 0) * 64 + lane] = hi;
      qs[(((w * NB + nb) * 4 + m) * 2 + 1) * 64 + lane] = lo;
    }
  }

  // This head's rows of the cache format in use (the other format's
  // pointers are null and stay untouched).
  const size_t gh = (size_t)g * a.Hkv + h;
  KVHead kv = {};
  kv.cap = a.cap;
  if constexpr (Q8) {
    kv.K8 = a.k8 + gh * a.cap * kD;
    kv.V8 = a.v8 + gh * kD * a.cap;
    kv.KS = a.ks + gh * a.cap * (kD / 32);
    kv.VS = a.vs + gh * (a.cap / 32) * kD;
  } else {
    kv.K = a.k + gh * a.cap * kD;
    kv.V = a.v + gh * kD * a.cap;
  }
  f4 acc[NB][8];
  float mrow[NB], lsum[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    mrow[nb] = -INFINITY;
    lsum[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[nb][db] = f4{0.f, 0.f, 0.f, 0.f};
  }

  for (int t0 = p0; t0 < p1; t0 += kTile) {
    KVTile x;
    load_tile<Q8>(kv, t0, Lg, col, grp, x);
    // q8_0: column blocks in pairs where they pair up, so that each code is
    // converted once per pair
    constexpr int NF = Q8 && NB % 2 == 0 ? 2 : 1;
#pragma unroll
    for (int nb = 0; nb < NB; nb += NF) {
      u4 qh[NF][4], ql[NF][4];
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          qh[f][m] = qs[(((w * NB + nb + f) * 4 + m) * 2 + 0) * 64 + lane];
          ql[f][m] = qs[(((w * NB + nb + f) * 4 + m) * 2 + 1) * 64 + lane];
        }
      tile_update_n<Q8, NF>(x, t0, Lg, lim + nb, grp, qh, ql, acc + nb, mrow + nb, lsum + nb);
    }
  }

  // Merge the block's splits: wave i's column max m_i, sums l_i and outputs
  // weigh 2^(m_i - max m); wave w then writes its share of the dimensions of
  // the block's partial.  Empty splits (m = -inf) weigh zero.
  __syncthreads();
  float* mb = smem;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float* dst = mb + (w * NB + nb) * kMergeFloats * 64 + lane;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(4 * db + i) * 64] = acc[nb][db][i];
    dst[32 * 64] = mrow[nb];
    dst[33 * 64] = lsum[nb];
  }
  __syncthreads();
  const int q4 = s >> 2;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float mi[kWaves], M = -INFINITY;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      mi[i] = mb[((i * NB + nb) * kMergeFloats + 32) * 64 + lane];
      M = fmaxf(M, mi[i]);
    }
    const float muse = M == -INFINITY ? 0.f : M;
    float wt[kWaves], l = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      wt[i] = exp2f(mi[i] - muse);
      l += wt[i] * mb[((i * NB + nb) * kMergeFloats + 33) * 64 + lane];
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int c = nb * 16 + col;
    if (c < NQ) {
      const int row = r0 + c / gqa, hq = h * gqa + c % gqa;
      const size_t base = ((size_t)row * a.Hq + hq) * a.smax + q4;
      float* po = a.part_o + base * kD + 4 * grp;
#pragma unroll
      for (int k = 0; k < 8 / kWaves; ++k) {
        const int db = (8 / kWaves) * w + k;
        f4 v = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
          const float* src = mb + ((i * NB + nb) * kMergeFloats + 4 * db) * 64 + lane;
          v += wt[i] * f4{src[0], src[64], src[128], src[192]};
        }
        *(f4*)(po + 16 * db) = v;
      }
      if (w == 0 && grp == 0) *(float2*)(a.part_ml + 2 * base) = make_float2(M, l);
    }
  }
}

// o[row][hq] = sum_q w_q o_q / sum_q w_q l_q with w_q = 2^(m_q - max m), then
// the output gate.  One block of 4 waves per (row, query head): wave w folds
// partials q = w, w+4, ... with a running max, each lane two dimensions; the
// four results merge through LDS.
__global__ __launch_bounds__(256) void k_attn_combine(const AttnArgs a) {
  __shared__ float red[kWaves][4][64];
  const int th = blockIdx.x, row = th / a.Hq, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int g = 0;
  while (row >= a.gs[g + 1]) ++g;
  const int nq = a.nsplit[g] / kWaves;
  const float2* ml = (const float2*)a.part_ml + (size_t)th * a.smax;
  const float* po = a.part_o + (size_t)th * a.smax * kD + 2 * lane;
  float m = -INFINITY, l = 0.f, y0 = 0.f, y1 = 0.f;
  for (int q = w; q < nq; q += kWaves) {
    const float2 v = ml[q];
    const float2 o = *(const float2*)(po + (size_t)q * kD);
    const float mn = fmaxf(m, v.x);
    if (mn == -INFINITY) continue;
    const float ao = exp2f(m - mn), aq = exp2f(v.x - mn);
    l = l * ao + v.y * aq;
    y0 = y0 * ao + o.x * aq;
    y1 = y1 * ao + o.y * aq;
    m = mn;
  }
  red[w][0][lane] = m;
  red[w][1][lane] = l;
  red[w][2][lane] = y0;
  red[w][3][lane] = y1;
  __syncthreads();
  if (w != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) M = fmaxf(M, red[i][0][lane]);
  float L = 0.f, z0 = 0.f, z1 = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const float wt = exp2f(red[i][0][lane] - M);
    L += wt * red[i][1][lane];
    z0 += wt * red[i][2][lane];
    z1 += wt * red[i][3][lane];
  }
  z0 /= L;
  z1 /= L;
  if (a.gate) {
    const float2 gt = *(const float2*)(a.gate + (size_t)th * kD + 2 * lane);
    z0 *= 1.f / (1.f + expf(-gt.x));
    z1 *= 1.f / (1.f + expf(-gt.y));
  }
  *(float2*)(a.o + (size_t)th * kD + 2 * lane) = make_float2(z0, z1);
}

}  // namespace

AttnPlan plan_attn(int G, const int32_t* ctx, const int32_t* gs, int Hkv, int cu_count, bool q8) {
  AttnPlan p = {};
  long W = 0, Lmax = 0;
  for (int g = 0; g < G; ++g) {
    const long L = (long)ctx[g] + (gs[g + 1] - gs[g]);
    W += L * Hkv;
    Lmax = L > Lmax ? L : Lmax;
  }
  // fp16 caches: about one wave per SIMD over the device (one block of four
  // per CU), at least four tiles per item unless the contexts are short, and
  // at most kAttnMaxSplit splits per head.  Measured on the 4 x 32768 and
  // 81920 workloads, four items per CU beat eight (the per-item set-up and
  // merge cost more than the second wave per SIMD gains), and 16 or 32 were
  // slower.  q8_0 caches carry half the bytes per position and more
  // arithmetic per byte, and take eight items per CU so that a second wave
  // per SIMD covers each wave's latency.
  const long target = (q8 ? 8L : 4L) * (cu_count > 0 ? cu_count : 256);
  auto up64 = [](long x) { return (x + kTile - 1) / kTile * kTile; };
  long chunk = up64((W + target - 1) / target);
  if (chunk < 4 * kTile) chunk = 4 * kTile;
  const long need = up64((Lmax + kAttnMaxSplit - 1) / kAttnMaxSplit);
  if (chunk < need) chunk = need;
  p.chunk = (int)chunk;
  p.item0[0] = 0;
  for (int g = 0; g < G; ++g) {
    const long L = (long)ctx[g] + (gs[g + 1] - gs[g]);
    p.nsplit[g] = (int)((L + chunk - 1) / chunk + kWaves - 1) / kWaves * kWaves;
    p.smax = p.nsplit[g] / kWaves > p.smax ? p.nsplit[g] / kWaves : p.smax;
    p.item0[g + 1] = p.item0[g] + p.nsplit[g] * Hkv;
  }
  p.n_items = p.item0[G];
  return p;
}

size_t attn_workspace_bytes(int T, int Hq, const AttnPlan& p) {
  const size_t n = (size_t)T * Hq * p.smax;
  return (n * kD * 4 + 255) / 256 * 256 + (n * 8 + 255) / 256 * 256;
}

hipError_t launch_attn(AttnArgs a, const AttnPlan& p, int nb, bool q8, void* ws, hipStream_t st) {
  const size_t n = (size_t)a.T * a.Hq * p.smax;
  a.part_o = (float*)ws;
  a.part_ml = (float*)((char*)ws + (n * kD * 4 + 255) / 256 * 256);
  a.chunk = p.chunk;
  a.smax = p.smax;
  a.n_items = p.n_items;
  for (int g = 0; g <= a.G; ++g) a.item0[g] = p.item0[g];
  for (int g = 0; g < a.G; ++g) a.nsplit[g] = p.nsplit[g];
  const dim3 grid(p.n_items / kWaves);
  switch (nb * 2 + (q8 ? 1 : 0)) {
    case 2: k_attn_split<1, false><<<grid, 256, 0, st>>>(a); break;
    case 3: k_attn_split<1, true><<<grid, 256, 0, st>>>(a); break;
    case 4: k_attn_split<2, false><<<grid, 256, 0, st>>>(a); break;
    case 5: k_attn_split<2, true><<<grid, 256, 0, st>>>(a); break;
    case 6: k_attn_split<3, false><<<grid, 256, 0, st>>>(a); break;
    case 7: k_attn_split<3, true><<<grid, 256, 0, st>>>(a); break;
    case 8: k_attn_split<4, false><<<grid, 256, 0, st>>>(a); break;
    case 9: k_attn_split<4, true><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_attn_combine<<<a.T * a.Hq, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mk
