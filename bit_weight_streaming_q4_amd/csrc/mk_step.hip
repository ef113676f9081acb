// mk_step.hip — one decode step in ONE persistent cooperative launch.
//
// Pages: richland.au single-stream article, "What shipped" (the whole cycle —
// main model over T = 1 + n_draft rows, lm_head and verification — runs in one
// persistent launch whose phases are separated by a software grid barrier;
// the host reads back only the accepted tokens; the Gated DeltaNet state is
// committed through the accepted token); richland.au 4-agent article, "Why it
// matters" (rows of several agents share one weight read per step).
//
// Phases of a step (a grid barrier after each):
//   prep       q8(x) and the per-tile sums of squares of x (RMSNorm input)
//   per layer  P_in    u  = r(x) * (P_in . q8(x))         -> q8(u)
//              P_out   x += P_out . q8(u)                  -> q8(x), sums of squares
//                      (+ Gated DeltaNet step per agent in GDN layers)
//              gate/up h  = SiLU(r g) * (r u)              -> q8(h)
//              down    x += W_down . q8(h)                 -> q8(x), sums of squares
//   lm_prep    hid = r(x) * x, split into fp16 hi + lo fragments
//   lm         logits, per-block argmax, last block: argmax, verify, accept
//              lengths into the GDN states for the next step's replay
// r(x)_t = 1/sqrt(mean(x_t^2) + 1e-6) multiplies the whole dot product of row
// t, so the GEMV runs on q8 of the un-normalised row and the factor is applied
// once in the epilogue.
//
// Work split: each GEMV phase is a line of "units" (64 output rows x one
// superblock = 9216 B of weights), tile-major; the participating waves take
// equal contiguous stretches of it (stream-K), computed arithmetically.  A
// wave flushes one fp32 partial per (tile, matrix) it touches; the last wave
// to flush a tile (atomic ticket) adds the partials in wave order and runs the
// epilogue, so results do not depend on timing.  GDN half-head jobs sit at the
// front of the P_out line with a weight of several units.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "mk.h"
#include "mk_device.h"
#include "mk_gdn.h"
#include "mk_internal.h"

namespace mk {

constexpr int kMaxAgents = 16;
constexpr int kMaxLayers = 128;
constexpr int kTicketTiles = 512;  // tickets per phase instance (max n_out / 64)
constexpr int kGdnHeadsPerLayer = 32;
constexpr int kGdnJobWeight = 7;  // a half-head job ~ 64 KB of state traffic ~ 7 units
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / 64;
constexpr float kRmsEps = 1e-6f;
constexpr unsigned kSpinLimit = 1u << 26;  // grid-barrier watchdog (~seconds)

enum { K_X = 0, K_U = 1, K_X2 = 2, K_H = 3 };

struct LayerW {
  const uint8_t* w[5];  // p_in, p_out, gate, up, down
};

struct StepArgs {
  int L, H, P, F, V, T, G;
  int gs[MK_LM_MAX_G + 1];
  int wp[5];    // participating waves per plan: P_in, P_out, gate/up, down, P_out+GDN
  int cmax[5];  // partial slots per (tile, matrix) per plan
  const LayerW* layers;
  const uint16_t* lm;
  uint64_t gdn_mask[2];
  int8_t gdn_idx[kMaxLayers];
  int n_agents, T_max, nh;
  float* S[kMaxAgents];
  float* ring[kMaxAgents];
  int32_t* nacc[kMaxAgents];
  const float *gq, *gk, *gv, *gg, *gb;
  float* go;
  float* x;
  float* trace;
  const int32_t* drafts;
  // workspace
  unsigned* bar;
  int* err;
  unsigned* tickets;
  unsigned* lm_ticket;
  int8_t* a8;
  float* ssg;
  size_t a8_layer, ssg_layer;
  size_t a8_off[4], ssg_off[4];
  float* ss;  // [(2L+1)][H/64][16]
  float* part;
  _Float16* frag;
  float* lm_val;
  int* lm_idx;
  int32_t* out;  // [0] error word, [16..31] n_acc, [32..47] tokens, [48..63] argmax
};

__device__ __forceinline__ bool layer_is_gdn(const StepArgs& a, int l) {
  return (a.gdn_mask[l >> 6] >> (l & 63)) & 1ull;
}

// Keeps loads through p from being issued before this point (the scalar-cache
// reads of a phase's activations must follow the grid barrier).
template <typename P>
__device__ __forceinline__ P* fresh(P* p) {
  asm volatile("" : "+s"(p)::"memory");
  return p;
}

// ------------------------------------------------------------ grid barrier
// Arrive: release fence, one atomic per block.  Wait: spin on the counter
// with an agent-scope load, then an acquire fence.  The counter only grows
// within a launch (zeroed before it), so barrier n waits for n * gridDim.x.
// A bounded spin sets the error word instead of hanging.
__device__ void grid_barrier(const StepArgs& a, unsigned& gen) {
  gen += gridDim.x;
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    atomicAdd(a.bar, 1u);
    unsigned spins = 0;
    while (__hip_atomic_load(a.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < gen) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        atomicOr(a.err, 1);
        break;
      }
    }
    __threadfence();
  }
  __syncthreads();
}

// ------------------------------------------------------------ work split
struct Split {
  long S;   // total weight of the phase line
  long Gw;  // weight of the GDN jobs at its front
  int W;    // participating waves
};

__device__ __forceinline__ long split_start(const Split& s, int w) { return (long)w * s.S / s.W; }
// wave whose stretch contains weight position p
__device__ __forceinline__ int wave_of_weight(const Split& s, long p) {
  return (int)(((p + 1) * (long)s.W - 1) / s.S);
}

// ------------------------------------------------------------ activations
struct ActRef {
  int8_t* a8;
  float* ssg;
  int K;
};

__device__ __forceinline__ ActRef act_ref(const StepArgs& a, int layer, int kind, int K) {
  ActRef r;
  r.a8 = a.a8 + (size_t)layer * a.a8_layer + a.a8_off[kind];
  r.ssg = a.ssg + (size_t)layer * a.ssg_layer + a.ssg_off[kind];
  r.K = K;
  return r;
}

// Quantizes, per row t < T, the 64 values val[t] (lane = column of tile tau)
// into the activation record; rows T..15 of the scale table get zeros.
template <int T>
__device__ __forceinline__ void store_q8(const ActRef& o, int tau, int lane, const float (&val)[T]) {
  const int g = 2 * tau + (lane >> 5);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const Q8 q = quant_group32(val[t]);
    o.a8[(size_t)t * o.K + (size_t)tau * 64 + lane] = (int8_t)q.a8;
    if ((lane & 31) == 0) {
      float* p = o.ssg + ((size_t)g * kTPad + t) * 2;
      p[0] = q.s;
      p[1] = q.s * (float)q.gsum;
    }
  }
  if ((lane & 31) == 0)
    for (int t = T; t < kTPad; ++t) {
      float* p = o.ssg + ((size_t)g * kTPad + t) * 2;
      p[0] = 0.0f;
      p[1] = 0.0f;
    }
}

// 1/sqrt(mean(x_t^2) + eps) from the per-tile sums of squares, for row t = lane
// (lanes >= T return 0); the sum runs over tiles in order.
__device__ __forceinline__ float rnorm_lane(const StepArgs& a, int ss_idx, int lane) {
  const int ntH = a.H / 64;
  float r = 0.0f;
  if (lane < a.T) {
    const float* ss = a.ss + (size_t)ss_idx * ntH * 16;
    float sum = 0.0f;
    for (int i = 0; i < ntH; ++i) sum += __builtin_nontemporal_load(ss + i * 16 + lane);
    r = 1.0f / __builtin_sqrtf(sum / (float)a.H + kRmsEps);
  }
  return r;
}

// Sum of squares of the 64 lanes' values (fixed butterfly order).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// ------------------------------------------------------------ GEMV phases
struct PhaseDesc {
  int ph, plan, layer, nm, K, N;
  const uint8_t* W[2];
  ActRef in;
  long gdn_jobs;
};

__device__ __forceinline__ PhaseDesc phase_desc(const StepArgs& a, int ph, int l) {
  PhaseDesc d;
  d.ph = ph;
  d.plan = ph;
  d.layer = l;
  // the weight table is written before the launch: scalar loads are safe
  const uint8_t* lw[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) lw[i] = *as_const<const uint8_t*>(&a.layers[l].w[i]);
  d.gdn_jobs = 0;
  switch (ph) {
    case 0:
      d.nm = 1, d.K = a.H, d.N = a.P, d.W[0] = lw[0], d.W[1] = lw[0];
      d.in = act_ref(a, l, K_X, a.H);
      break;
    case 1:
      d.nm = 1, d.K = a.P, d.N = a.H, d.W[0] = lw[1], d.W[1] = lw[1];
      d.in = act_ref(a, l, K_U, a.P);
      if (a.n_agents > 0 && layer_is_gdn(a, l)) {
        d.gdn_jobs = (long)a.n_agents * kGdnHeadsPerLayer * 2;
        d.plan = 4;
      }
      break;
    case 2:
      d.nm = 2, d.K = a.H, d.N = a.F, d.W[0] = lw[2], d.W[1] = lw[3];
      d.in = act_ref(a, l, K_X2, a.H);
      break;
    default:
      d.nm = 1, d.K = a.F, d.N = a.H, d.W[0] = lw[4], d.W[1] = lw[4];
      d.in = act_ref(a, l, K_H, a.F);
      break;
  }
  return d;
}

// Sum of the partials of (tile, matrix) tm, in contributing-wave order.
template <int T>
__device__ __forceinline__ void sum_partials(const StepArgs& a, const PhaseDesc& d, const Split& sp, int nsb,
                                             int tm, int lane, float (&v)[T]) {
  const long u0 = (long)tm * nsb;
  const int lo = wave_of_weight(sp, sp.Gw + u0), hi = wave_of_weight(sp, sp.Gw + u0 + nsb - 1);
  const float* base = a.part + ((size_t)tm * a.cmax[d.plan]) * T * 64;
#pragma unroll
  for (int t = 0; t < T; ++t) v[t] = 0.0f;
  for (int c = 0; c <= hi - lo; ++c)
#pragma unroll
    for (int t = 0; t < T; ++t) v[t] += __builtin_nontemporal_load(base + ((size_t)c * T + t) * 64 + lane);
}

template <int T>
__device__ void epilogue(const StepArgs& a, const PhaseDesc& d, const Split& sp, int nsb, int tau, int lane) {
  float v0[T], v1[T];
  sum_partials<T>(a, d, sp, nsb, tau * d.nm, lane, v0);
  if (d.nm == 2) sum_partials<T>(a, d, sp, nsb, tau * 2 + 1, lane, v1);
  const int l = d.layer;
  const int col = tau * 64 + lane;
  if (d.ph == 0 || d.ph == 2) {
    const float rl = rnorm_lane(a, d.ph == 0 ? 2 * l : 2 * l + 1, lane);
    float y[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float r = __shfl(rl, t, 64);
      if (d.ph == 0) {
        y[t] = r * v0[t];
      } else {
        const float g = r * v0[t], u = r * v1[t];
        y[t] = g * u / (1.0f + expf(-g));
      }
    }
    store_q8<T>(act_ref(a, l, d.ph == 0 ? K_U : K_H, d.ph == 0 ? a.P : a.F), tau, lane, y);
  } else {
    float xn[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float* xp = a.x + (size_t)t * a.H + col;
      xn[t] = *xp + v0[t];
      *xp = xn[t];
    }
    const int ss_idx = d.ph == 1 ? 2 * l + 1 : 2 * l + 2;
    float* ss = a.ss + ((size_t)ss_idx * (a.H / 64) + tau) * 16;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s2 = wave_sum(xn[t] * xn[t]);
      if (lane == 0) ss[t] = s2;
    }
    if (d.ph == 3 && a.trace) {
#pragma unroll
      for (int t = 0; t < T; ++t) a.trace[((size_t)l * T + t) * a.H + col] = xn[t];
    }
    if (d.ph == 1)
      store_q8<T>(act_ref(a, l, K_X2, a.H), tau, lane, xn);
    else if (l + 1 < a.L)
      store_q8<T>(act_ref(a, l + 1, K_X, a.H), tau, lane, xn);
  }
}

__device__ void gdn_job(const StepArgs& a, int layer, long j, int lane) {
  const int agent = (int)(j / (kGdnHeadsPerLayer * 2));
  const int head = (int)((j / 2) % kGdnHeadsPerLayer);
  const int half = (int)(j & 1);
  // per-agent values indexed from the argument block: make them wave-uniform
  const int hh = uniform((int)a.gdn_idx[layer]) * kGdnHeadsPerLayer + head;
  const int32_t* na = uniform(a.nacc[agent]);
  const int par = *as_const<int32_t>(na + 1) & 1;
  const int r0 = uniform(a.gs[agent]);
  const int r1 = uniform(a.gs[agent + 1]);
  float* const Sa = uniform(a.S[agent]);
  float* const Ra = uniform(a.ring[agent]);
  GdnHalf x;
  x.S = Sa + (size_t)hh * kD * kD;
  x.ring_rd = Ra + ((size_t)par * a.nh + hh) * (a.T_max - 1) * kRingRow;
  x.ring_wr = Ra + ((size_t)(par ^ 1) * a.nh + hh) * (a.T_max - 1) * kRingRow;
  x.nrep = clamp_acc(*as_const<int32_t>(na), a.T_max);
  x.q = a.gq + ((size_t)r0 * a.nh + hh) * kD;
  x.k = a.gk + ((size_t)r0 * a.nh + hh) * kD;
  x.v = a.gv + ((size_t)r0 * a.nh + hh) * kD;
  x.g = a.gg + (size_t)r0 * a.nh + hh;
  x.beta = a.gb + (size_t)r0 * a.nh + hh;
  x.sqk = (size_t)a.nh * kD;
  x.sv = (size_t)a.nh * kD;
  x.sgb = a.nh;
  x.o = a.go + ((size_t)r0 * a.nh + hh) * kD;
  x.so = (size_t)a.nh * kD;
  x.T = r1 - r0;
  x.half = half;
  gdn_half_step(x, lane);
}

template <int T>
__device__ void gemv_phase(const StepArgs& a, const PhaseDesc& d, int w, int lane) {
  const int nsb = d.K / 256;
  const int ntiles = d.N / 64;
  Split sp;
  sp.Gw = d.gdn_jobs * kGdnJobWeight;
  sp.S = sp.Gw + (long)ntiles * d.nm * nsb;
  sp.W = a.wp[d.plan];
  if (w >= sp.W) return;
  const long s0 = split_start(sp, w), s1 = split_start(sp, w + 1);
  // Gated DeltaNet jobs whose start falls in this stretch
  for (long j = (s0 + kGdnJobWeight - 1) / kGdnJobWeight; j * kGdnJobWeight < s1 && j < d.gdn_jobs; ++j)
    gdn_job(a, d.layer, j, lane);
  QAct act;
  act.a8 = fresh(d.in.a8);
  act.ssg = fresh(d.in.ssg);
  act.K = d.K;
  act.T = T;
  long u = (s0 > sp.Gw ? s0 : sp.Gw) - sp.Gw;
  const long u1 = (s1 > sp.Gw ? s1 : sp.Gw) - sp.Gw;
  unsigned* tickets = a.tickets + ((size_t)d.layer * 4 + d.ph) * kTicketTiles;
  while (u < u1) {
    const int tm = (int)(u / nsb);
    const int b0 = (int)(u % nsb);
    const int len = (int)((u1 - u) < (long)(nsb - b0) ? (u1 - u) : (long)(nsb - b0));
    const int tau = tm / d.nm, m = tm % d.nm;
    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = 0.0f;
    dot4_range<T>(d.W[m] + (size_t)tau * nsb * kUnitBytes, b0, b0 + len, act, lane, acc);
    const int lo = wave_of_weight(sp, sp.Gw + (long)tm * nsb);
    float* dst = a.part + ((size_t)tm * a.cmax[d.plan] + (w - lo)) * T * 64;
#pragma unroll
    for (int t = 0; t < T; ++t) dst[t * 64 + lane] = acc[t];
    // ticket: the last contribution to this tile runs its epilogue
    int expect = 0;
    for (int mm = 0; mm < d.nm; ++mm) {
      const long uu = ((long)tau * d.nm + mm) * nsb;
      expect += wave_of_weight(sp, sp.Gw + uu + nsb - 1) - wave_of_weight(sp, sp.Gw + uu) + 1;
    }
    unsigned prev = 0;
    if (lane == 0) {
      __threadfence();
      prev = atomicAdd(tickets + tau, 1u);
    }
    prev = __shfl(prev, 0, 64);
    if ((int)prev == expect - 1) {
      __threadfence();
      epilogue<T>(a, d, sp, nsb, tau, lane);
    }
    u += len;
  }
}

// ------------------------------------------------------------ small phases
template <int T>
__device__ void prep_phase(const StepArgs& a, int w, int lane, int nw) {
  const int ntH = a.H / 64;
  for (int tau = w; tau < ntH; tau += nw) {
    float xv[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xv[t] = a.x[(size_t)t * a.H + tau * 64 + lane];
    float* ss = a.ss + (size_t)tau * 16;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s2 = wave_sum(xv[t] * xv[t]);
      if (lane == 0) ss[t] = s2;
    }
    store_q8<T>(act_ref(a, 0, K_X, a.H), tau, lane, xv);
  }
}

__device__ void lm_prep_phase(const StepArgs& a, int w, int lane, int nw) {
  const int nc = a.H / 64;
  const int t = lane & 15, kq = lane >> 4;
  const float rl = rnorm_lane(a, 2 * a.L, lane);
  const float r = __shfl(rl, t, 64);
  for (int c = w; c < nc; c += nw) {
    _Float16* o = a.frag + ((size_t)c * 64 + lane) * 32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float xv = t < a.T ? r * a.x[(size_t)t * a.H + 64 * c + 16 * kq + e] : 0.0f;
      const _Float16 hi = (_Float16)xv;
      o[e] = hi;
      o[16 + e] = (_Float16)(xv - (float)hi);
    }
  }
}

__device__ __forceinline__ bool lm_better(float va, int ia, float vb, int ib) {
  if (ia < 0) return false;
  if (ib < 0) return true;
  if (va != va) return false;
  if (vb != vb) return true;
  return va > vb || (va == vb && ia < ib);
}

__device__ void lm_phase(const StepArgs& a) {
  __shared__ float red[4][64][16];
  __shared__ int last;
  __shared__ int fin[16];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int vl = l & 15, kq = l >> 4;
  const int nc = a.H / 64;
  const int c0 = (nc * w) / 4, c1 = (nc * (w + 1)) / 4;
  const int nblk = (a.V + 63) / 64;
  const int t_own = threadIdx.x >> 4, part = threadIdx.x & 15;
  float best = 0.0f;
  int bidx = -1;
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int v0 = blk * 64;
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
          const u32x4* wpp = (const u32x4*)(a.lm + (size_t)v * a.H + 64 * c + 16 * kq);
          wa[g][0] = __builtin_nontemporal_load(wpp);
          wa[g][1] = __builtin_nontemporal_load(wpp + 1);
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
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w][16 * g + 4 * kq + i][vl] = acc[g][i];
    __syncthreads();
    for (int r = 4 * part; r < 4 * part + 4; ++r) {
      const int v = v0 + r;
      if (v >= a.V) break;
      const float xv = ((red[0][r][t_own] + red[1][r][t_own]) + red[2][r][t_own]) + red[3][r][t_own];
      if (lm_better(xv, v, best, bidx)) {
        best = xv;
        bidx = v;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(best, m, 16);
    const int oi = __shfl_xor(bidx, m, 16);
    if (lm_better(ov, oi, best, bidx)) {
      best = ov;
      bidx = oi;
    }
  }
  if (part == 0) {
    a.lm_val[(size_t)blockIdx.x * 16 + t_own] = best;
    a.lm_idx[(size_t)blockIdx.x * 16 + t_own] = bidx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    last = (atomicAdd(a.lm_ticket, 1u) == gridDim.x - 1);
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  best = 0.0f;
  bidx = -1;
  for (int b = part; b < (int)gridDim.x; b += 16) {
    const float xv = __builtin_nontemporal_load(a.lm_val + (size_t)b * 16 + t_own);
    const int iv = __builtin_nontemporal_load(a.lm_idx + (size_t)b * 16 + t_own);
    if (lm_better(xv, iv, best, bidx)) {
      best = xv;
      bidx = iv;
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(best, m, 16);
    const int oi = __shfl_xor(bidx, m, 16);
    if (lm_better(ov, oi, best, bidx)) {
      best = ov;
      bidx = oi;
    }
  }
  if (part == 0) fin[t_own] = bidx;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int t = 0; t < a.T; ++t) a.out[48 + t] = fin[t];
    for (int g = 0; g < a.G; ++g) {
      const int r = a.gs[g], n = a.gs[g + 1] - a.gs[g];
      const int32_t* dr = a.drafts + (r - g);
      int k = 0;
      while (k < n - 1 && fin[r + k] >= 0 && dr[k] == fin[r + k]) ++k;
      a.out[16 + g] = k;
      for (int i = 0; i < n; ++i) a.out[32 + r + i] = i < k ? dr[i] : (i == k ? fin[r + k] : -1);
      if (g < a.n_agents) {
        a.nacc[g][0] = k;      // replayed by the next step
        a.nacc[g][1] ^= 1;     // this step's rows are in the other ring half
      }
    }
  }
}

// ------------------------------------------------------------ the kernel
template <int T>
__global__ __launch_bounds__(kBlock) void k_decode_step(StepArgs a) {
  const int lane = threadIdx.x & 63;
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x * kWavesPerBlock + wib;
  const int nw = gridDim.x * kWavesPerBlock;
  unsigned gen = 0;
  prep_phase<T>(a, w, lane, nw);
  grid_barrier(a, gen);
  for (int l = 0; l < a.L; ++l) {
    for (int ph = 0; ph < 4; ++ph) {
      const PhaseDesc d = phase_desc(a, ph, l);
      gemv_phase<T>(a, d, w, lane);
      grid_barrier(a, gen);
    }
  }
  lm_prep_phase(a, w, lane, nw);
  grid_barrier(a, gen);
  lm_phase(a);
}

// ------------------------------------------------------------ host side
typedef void (*StepKernel)(StepArgs);

template <int T>
static StepKernel kernel_for() {
  return k_decode_step<T>;
}

static StepKernel step_kernel(int T) {
  switch (T) {
    case 1: return kernel_for<1>();
    case 2: return kernel_for<2>();
    case 3: return kernel_for<3>();
    case 4: return kernel_for<4>();
    case 5: return kernel_for<5>();
    case 6: return kernel_for<6>();
    case 7: return kernel_for<7>();
    case 8: return kernel_for<8>();
    case 9: return kernel_for<9>();
    case 10: return kernel_for<10>();
    case 11: return kernel_for<11>();
    case 12: return kernel_for<12>();
    case 13: return kernel_for<13>();
    case 14: return kernel_for<14>();
    case 15: return kernel_for<15>();
    case 16: return kernel_for<16>();
    default: return nullptr;
  }
}

}  // namespace mk

using namespace mk;

struct mk_stack {
  mk_stack_desc d;
  std::vector<LayerW> layers;
  std::vector<mk_deltanet> dn;
  std::vector<uint8_t> gdn_flag;
  int n_gdn_layers = 0;
  int8_t gdn_idx[kMaxLayers];
  void* uploaded_ws = nullptr;  // workspace that holds the current weight table
};

namespace {

size_t a256(size_t n) { return (n + 255) / 256 * 256; }

struct StepLayout {
  int grid, waves;
  int wp[5], cmax[5];
  size_t off_ctrl, n_ctrl;  // zeroed before each launch: barrier, tickets
  size_t off_out, off_tickets, off_lmticket, off_table, off_a8, off_ssg, off_ss, off_part, off_frag, off_lmv,
      off_lmi, total;
  size_t a8_layer, ssg_layer, a8_off[4], ssg_off[4];
};

int host_wave_of(long S, int W, long p) { return (int)(((p + 1) * (long)W - 1) / S); }

// Participating waves and the largest number of partials a (tile, matrix)
// receives, for one GEMV phase.
void plan_phase(long units_tiles, int nm, int nsb, long gdn_w, int waves, int& wp, int& cmax) {
  const long S = gdn_w + units_tiles * nm * nsb;
  // at least one unit per participating wave, and at least ~1.5 on average
  long want = S * 2 / 3;
  if (want < 1) want = 1;
  wp = (int)std::min<long>(waves, std::min<long>(want, S));
  cmax = 1;
  for (long tm = 0; tm < units_tiles * nm; ++tm) {
    const long u0 = gdn_w + tm * nsb;
    const int c = host_wave_of(S, wp, u0 + nsb - 1) - host_wave_of(S, wp, u0) + 1;
    cmax = std::max(cmax, c);
  }
}

StepLayout layout(const mk_stack* st, int T) {
  StepLayout y;
  const mk_stack_desc& d = st->d;
  int dev = 0, cu = 256;
  hipGetDevice(&dev);
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) == hipSuccess) cu = p.multiProcessorCount;
  int per_cu = 0;
  StepKernel k = step_kernel(T);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k, kBlock, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  per_cu = std::min(per_cu, 4);
  y.grid = cu * per_cu;
  y.waves = y.grid * kWavesPerBlock;
  const int n_agents = st->dn.empty() ? 0 : d.n_agents;
  const long gdn_w = (long)n_agents * kGdnHeadsPerLayer * 2 * kGdnJobWeight;
  plan_phase(d.proj / 64, 1, d.hidden / 256, 0, y.waves, y.wp[0], y.cmax[0]);
  plan_phase(d.hidden / 64, 1, d.proj / 256, 0, y.waves, y.wp[1], y.cmax[1]);
  plan_phase(d.ffn / 64, 2, d.hidden / 256, 0, y.waves, y.wp[2], y.cmax[2]);
  plan_phase(d.hidden / 64, 1, d.ffn / 256, 0, y.waves, y.wp[3], y.cmax[3]);
  plan_phase(d.hidden / 64, 1, d.proj / 256, gdn_w, y.waves, y.wp[4], y.cmax[4]);
  y.a8_off[K_X] = 0;
  y.a8_off[K_U] = a256((size_t)T * d.hidden);
  y.a8_off[K_X2] = y.a8_off[K_U] + a256((size_t)T * d.proj);
  y.a8_off[K_H] = y.a8_off[K_X2] + a256((size_t)T * d.hidden);
  y.a8_layer = y.a8_off[K_H] + a256((size_t)T * d.ffn);
  auto sgb = [](int K) { return a256((size_t)(K / 32) * kTPad * 8); };
  y.ssg_off[K_X] = 0;
  y.ssg_off[K_U] = sgb(d.hidden);
  y.ssg_off[K_X2] = y.ssg_off[K_U] + sgb(d.proj);
  y.ssg_off[K_H] = y.ssg_off[K_X2] + sgb(d.hidden);
  y.ssg_layer = y.ssg_off[K_H] + sgb(d.ffn);
  size_t o = 0;
  y.off_ctrl = o;
  o += 256;  // barrier counter
  y.off_lmticket = o;
  o += 256;
  y.off_tickets = o;
  o += a256((size_t)d.n_layers * 4 * kTicketTiles * 4);
  y.n_ctrl = o - y.off_ctrl;
  y.off_out = o;
  o += 256;
  y.off_table = o;
  o += a256(sizeof(LayerW) * d.n_layers);
  y.off_a8 = o;
  o += y.a8_layer * d.n_layers;
  y.off_ssg = o;
  o += y.ssg_layer * d.n_layers;
  y.off_ss = o;
  o += a256((size_t)(2 * d.n_layers + 1) * (d.hidden / 64) * 16 * 4);
  y.off_part = o;
  size_t part = 0;
  const int tiles[5] = {d.proj / 64, d.hidden / 64, d.ffn / 64, d.hidden / 64, d.hidden / 64};
  const int nms[5] = {1, 1, 2, 1, 1};
  for (int i = 0; i < 5; ++i) part = std::max(part, (size_t)tiles[i] * nms[i] * y.cmax[i] * T * 64 * 4);
  o += a256(part);
  y.off_frag = o;
  o += a256((size_t)(d.hidden / 64) * 64 * 32 * 2);
  y.off_lmv = o;
  o += a256((size_t)y.grid * 16 * 4);
  y.off_lmi = o;
  o += a256((size_t)y.grid * 16 * 4);
  y.total = o;
  return y;
}

int sfail(int status, const char* msg) { return set_error(status, "%s", msg); }

int valid_q(const mk_q4k& w, int n_out, int n_in) {
  return w.blocks && w.n_out == n_out && w.n_in == n_in && ((uintptr_t)w.blocks % 256) == 0;
}

}  // namespace

extern "C" {

int mk_stack_create(const mk_stack_desc* desc, mk_stack** out) {
  if (!desc || !out) return sfail(MK_ERR_ARG, "stack: null argument");
  *out = nullptr;
  const mk_stack_desc& d = *desc;
  if (d.n_layers < 1 || d.n_layers > kMaxLayers) return sfail(MK_ERR_RANGE, "stack: n_layers outside 1..128");
  if (d.hidden <= 0 || d.proj <= 0 || d.ffn <= 0 || d.hidden % 256 || d.proj % 256 || d.ffn % 256)
    return sfail(MK_ERR_SHAPE, "stack: hidden, proj, ffn must be positive multiples of 256");
  if (d.hidden > 64 * kTicketTiles || d.proj > 64 * kTicketTiles || d.ffn > 64 * kTicketTiles)
    return sfail(MK_ERR_SHAPE, "stack: widths above 32768");
  if (d.vocab <= 0 || !d.lm_head || ((uintptr_t)d.lm_head % 16))
    return sfail(MK_ERR_ARG, "stack: lm_head missing or misaligned");
  if (!d.p_in || !d.p_out || !d.gate || !d.up || !d.down) return sfail(MK_ERR_ARG, "stack: null weight array");
  mk_stack* st = new mk_stack();
  st->d = d;
  st->layers.resize(d.n_layers);
  for (int l = 0; l < d.n_layers; ++l) {
    if (!valid_q(d.p_in[l], d.proj, d.hidden) || !valid_q(d.p_out[l], d.hidden, d.proj) ||
        !valid_q(d.gate[l], d.ffn, d.hidden) || !valid_q(d.up[l], d.ffn, d.hidden) ||
        !valid_q(d.down[l], d.hidden, d.ffn)) {
      delete st;
      return sfail(MK_ERR_SHAPE, "stack: a layer weight has the wrong shape, is null or misaligned");
    }
    const mk_q4k* ws[5] = {&d.p_in[l], &d.p_out[l], &d.gate[l], &d.up[l], &d.down[l]};
    for (int i = 0; i < 5; ++i) st->layers[l].w[i] = (const uint8_t*)ws[i]->blocks;
  }
  memset(st->gdn_idx, -1, sizeof(st->gdn_idx));
  st->gdn_flag.assign(d.n_layers, 0);
  if (d.h_gdn_layer)
    for (int l = 0; l < d.n_layers; ++l)
      if (d.h_gdn_layer[l]) {
        st->gdn_flag[l] = 1;
        st->gdn_idx[l] = (int8_t)st->n_gdn_layers++;
      }
  if (st->n_gdn_layers) {
    if (d.n_agents < 1 || d.n_agents > kMaxAgents || !d.dn) {
      delete st;
      return sfail(MK_ERR_ARG, "stack: GDN layers need 1..16 agent states");
    }
    for (int g = 0; g < d.n_agents; ++g) {
      const mk_deltanet& s = d.dn[g];
      if (!s.S || !s.ring || !s.n_acc || s.dk != 128 || s.dv != 128 ||
          s.nh != st->n_gdn_layers * kGdnHeadsPerLayer || s.T_max < 2 || s.T_max > MK_T_MAX) {
        delete st;
        return sfail(MK_ERR_SHAPE, "stack: agent state must have dk = dv = 128 and nh = gdn layers * 32");
      }
      st->dn.push_back(s);
    }
  }
  *out = st;
  return MK_OK;
}

void mk_stack_destroy(mk_stack* st) { delete st; }

size_t mk_decode_step_workspace(const mk_stack* st, int32_t T) {
  if (!st || T < 1 || T > MK_T_MAX) return 0;
  return layout(st, T).total;
}

int mk_decode_step(mk_stack* st, float* x, int32_t T, const int32_t* h_group_start, int32_t G,
                   const int32_t* drafts, const float* gdn_q, const float* gdn_k, const float* gdn_v,
                   const float* gdn_g, const float* gdn_beta, float* gdn_o, int32_t* h_tokens, int32_t* h_n_acc,
                   int32_t* d_argmax, float* trace, void* ws, size_t ws_bytes, void* stream) {
  if (!st) return sfail(MK_ERR_ARG, "decode: null stack");
  if (T < 1 || T > MK_T_MAX) return sfail(MK_ERR_RANGE, "decode: T outside 1..16");
  if (!x || ((uintptr_t)x % 16)) return sfail(MK_ERR_ALIGN, "decode: x null or misaligned");
  if (!h_tokens || !h_n_acc) return sfail(MK_ERR_ARG, "decode: null host output");
  std::vector<int> gs;
  if (!h_group_start) {
    if (G != 1) return sfail(MK_ERR_ARG, "decode: h_group_start null but G != 1");
    gs = {0, T};
  } else {
    if (G < 1 || G > MK_LM_MAX_G || G > T) return sfail(MK_ERR_RANGE, "decode: G outside 1..min(T, 16)");
    gs.assign(h_group_start, h_group_start + G + 1);
    if (gs[0] != 0 || gs[G] != T) return sfail(MK_ERR_RANGE, "decode: group starts must run from 0 to T");
    for (int g = 0; g < G; ++g)
      if (gs[g + 1] <= gs[g]) return sfail(MK_ERR_RANGE, "decode: empty group");
  }
  if (T > G && !drafts) return sfail(MK_ERR_ARG, "decode: drafts null");
  const bool gdn = st->n_gdn_layers > 0;
  if (gdn) {
    if (G != (int)st->dn.size()) return sfail(MK_ERR_ARG, "decode: G must equal the number of agent states");
    if (!gdn_q || !gdn_k || !gdn_v || !gdn_g || !gdn_beta || !gdn_o)
      return sfail(MK_ERR_ARG, "decode: GDN inputs/outputs missing");
    for (int g = 0; g < G; ++g)
      if (gs[g + 1] - gs[g] > st->dn[g].T_max) return sfail(MK_ERR_RANGE, "decode: group longer than its T_max");
  }
  const StepLayout y = layout(st, T);
  if (!ws || ws_bytes < y.total) return set_error(MK_ERR_WORKSPACE, "decode: workspace %zu < %zu bytes", ws_bytes, y.total);
  if ((uintptr_t)ws % 256) return sfail(MK_ERR_ALIGN, "decode: workspace not 256-B aligned");
  hipStream_t s = (hipStream_t)stream;
  uint8_t* w8 = (uint8_t*)ws;
  if (st->uploaded_ws != ws) {
    if (hipMemcpyAsync(w8 + y.off_table, st->layers.data(), sizeof(LayerW) * st->layers.size(),
                       hipMemcpyHostToDevice, s) != hipSuccess)
      return sfail(MK_ERR_LAUNCH, "decode: weight table upload failed");
    st->uploaded_ws = ws;
  }
  if (hipMemsetAsync(w8 + y.off_ctrl, 0, y.n_ctrl, s) != hipSuccess ||
      hipMemsetAsync(w8 + y.off_out, 0, 256, s) != hipSuccess)
    return sfail(MK_ERR_LAUNCH, "decode: control reset failed");
  StepArgs a;
  memset(&a, 0, sizeof(a));
  const mk_stack_desc& d = st->d;
  a.L = d.n_layers;
  a.H = d.hidden;
  a.P = d.proj;
  a.F = d.ffn;
  a.V = d.vocab;
  a.T = T;
  a.G = G;
  for (int i = 0; i <= MK_LM_MAX_G; ++i) a.gs[i] = i <= G ? gs[i] : T;
  for (int i = 0; i < 5; ++i) {
    a.wp[i] = y.wp[i];
    a.cmax[i] = y.cmax[i];
  }
  a.layers = (const LayerW*)(w8 + y.off_table);
  a.lm = d.lm_head;
  for (int l = 0; l < d.n_layers; ++l)
    if (st->gdn_flag[l]) a.gdn_mask[l >> 6] |= 1ull << (l & 63);
  memcpy(a.gdn_idx, st->gdn_idx, sizeof(a.gdn_idx));
  a.n_agents = gdn ? G : 0;
  if (gdn) {
    a.T_max = st->dn[0].T_max;
    a.nh = st->dn[0].nh;
    for (int g = 0; g < G; ++g) {
      if (st->dn[g].T_max != a.T_max) return sfail(MK_ERR_ARG, "decode: agent states need one T_max");
      a.S[g] = st->dn[g].S;
      a.ring[g] = st->dn[g].ring;
      a.nacc[g] = st->dn[g].n_acc;
    }
  }
  a.gq = gdn_q;
  a.gk = gdn_k;
  a.gv = gdn_v;
  a.gg = gdn_g;
  a.gb = gdn_beta;
  a.go = gdn_o;
  a.x = x;
  a.trace = trace;
  a.drafts = drafts;
  a.bar = (unsigned*)(w8 + y.off_ctrl);
  a.lm_ticket = (unsigned*)(w8 + y.off_lmticket);
  a.tickets = (unsigned*)(w8 + y.off_tickets);
  a.out = (int32_t*)(w8 + y.off_out);
  a.err = a.out;
  a.a8 = (int8_t*)(w8 + y.off_a8);
  a.ssg = (float*)(w8 + y.off_ssg);
  a.a8_layer = y.a8_layer;
  a.ssg_layer = y.ssg_layer / 4;
  for (int i = 0; i < 4; ++i) {
    a.a8_off[i] = y.a8_off[i];
    a.ssg_off[i] = y.ssg_off[i] / 4;
  }
  a.ss = (float*)(w8 + y.off_ss);
  a.part = (float*)(w8 + y.off_part);
  a.frag = (_Float16*)(w8 + y.off_frag);
  a.lm_val = (float*)(w8 + y.off_lmv);
  a.lm_idx = (int*)(w8 + y.off_lmi);
  void* args[] = {&a};
  hipError_t e = hipLaunchCooperativeKernel((const void*)step_kernel(T), dim3(y.grid), dim3(kBlock), args, 0, s);
  if (e != hipSuccess)
    return set_error(e == hipErrorCooperativeLaunchTooLarge ? MK_ERR_COOP : MK_ERR_LAUNCH,
                     "decode: cooperative launch failed: %s", hipGetErrorString(e));
  if (d_argmax &&
      hipMemcpyAsync(d_argmax, w8 + y.off_out + 48 * 4, T * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return sfail(MK_ERR_LAUNCH, "decode: argmax copy failed");
  int32_t hout[64];
  if (hipMemcpyAsync(hout, w8 + y.off_out, sizeof(hout), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return sfail(MK_ERR_LAUNCH, "decode: readback failed");
  if (hout[0]) return sfail(MK_ERR_DEVICE, "decode: grid-barrier watchdog fired");
  for (int g = 0; g < G; ++g) h_n_acc[g] = hout[16 + g];
  for (int t = 0; t < T; ++t) h_tokens[t] = hout[32 + t];
  set_error(MK_OK, "");
  return MK_OK;
}

}  // extern "C"
