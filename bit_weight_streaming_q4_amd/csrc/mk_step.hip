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
constexpr int kTicketStride = 16;  // counters 64 B apart
constexpr int kGdnHeadsPerLayer = 32;
constexpr int kGdnJobWeight = 7;  // a half-head job ~ 64 KB of state traffic ~ 7 units
constexpr int kBlock = 512;
constexpr int kWavesPerBlock = kBlock / 64;
constexpr float kRmsEps = 1e-6f;
constexpr unsigned kSpinLimit = 1u << 26;  // grid-barrier watchdog (~seconds)
constexpr int kMaxStamps = 4 * kMaxLayers + 8;

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
  uint64_t* stamps;  // [kMaxStamps]: block 0's clock after each barrier
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

// Cross-workgroup data of a step (partials, residual, sums of squares,
// activations) is stored and loaded with device-scope (sc1) accesses, which
// are coherent across the XCDs' L2 caches without whole-cache write-back or
// invalidation; ordering comes from waiting for the stores (workgroup-scope
// release) before the ticket/barrier atomic.  Activations are read through
// the scalar cache: every activation buffer is written once per launch and
// only read after its producer phase, so no stale line can be cached.
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh_i8(int8_t* p, int8_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_coh_i(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ticket_add(unsigned* p) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // this wave's stores have completed
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ grid barrier
// Arrive: one device-scope atomic per block once all its waves' stores have
// completed.  Wait: spin on the counter with device-scope loads.  The counter
// only grows within a launch (zeroed before it), so barrier n waits for
// n * gridDim.x.  A bounded spin sets the error word instead of hanging, and
// every later barrier then falls through.
__device__ void grid_barrier(const StepArgs& a, unsigned& gen) {
  const int idx = gen / gridDim.x;
  gen += gridDim.x;
  __syncthreads();  // every wave of the block has completed its stores
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(a.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned spins = 0;
    while (__hip_atomic_load(a.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < gen) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit || __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        atomicOr(a.err, 1);
        break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (blockIdx.x == 0 && idx + 1 < kMaxStamps) a.stamps[idx + 1] = wall_clock64();
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
    st_coh_i8(o.a8 + (size_t)t * o.K + (size_t)tau * 64 + lane, (int8_t)q.a8);
    if ((lane & 31) == 0) {
      float* p = o.ssg + ((size_t)g * kTPad + t) * 2;
      st_coh(p, q.s);
      st_coh(p + 1, q.s * (float)q.gsum);
    }
  }
  if ((lane & 31) == 0)
    for (int t = T; t < kTPad; ++t) {
      float* p = o.ssg + ((size_t)g * kTPad + t) * 2;
      st_coh(p, 0.0f);
      st_coh(p + 1, 0.0f);
    }
}

// 1/sqrt(mean(x_t^2) + eps) from the per-tile sums of squares, for row t = lane
// (lanes >= T return 0); the sum runs over tiles in order.
__device__ __forceinline__ float rnorm_lane(const StepArgs& a, int ss_idx, int lane) {
  const int ntH = uniform(a.H / 64);
  const int tl = lane < a.T ? lane : 0;  // every lane loads (in range); lanes >= T are discarded
  const float* ss = a.ss + (size_t)ss_idx * ntH * 16 + tl;
  float sum = 0.0f;
  for (int i0 = 0; i0 < ntH; i0 += 16) {
    float tmp[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) tmp[i] = ld_coh(ss + (size_t)(i0 + i < ntH ? i0 + i : ntH - 1) * 16);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i0 + i < ntH) sum += tmp[i];
  }
  return lane < a.T ? 1.0f / __builtin_sqrtf(sum / (float)a.H + kRmsEps) : 0.0f;
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

// Sum of the partials of (tile, matrix) tm, in contributing-wave order.  The
// device-scope loads are issued in batches of 4 partials so their latencies
// overlap (a loop of single loads waits for each one).
template <int T>
__device__ __forceinline__ void sum_partials(const StepArgs& a, const PhaseDesc& d, const Split& sp, int nsb,
                                             int tm, int lane, float (&v)[T]) {
  const long u0 = (long)tm * nsb;
  const int lo = wave_of_weight(sp, sp.Gw + u0), hi = wave_of_weight(sp, sp.Gw + u0 + nsb - 1);
  const int n = uniform(hi - lo + 1);
  const float* base = a.part + ((size_t)tm * a.cmax[d.plan]) * T * 64 + lane;
#pragma unroll
  for (int t = 0; t < T; ++t) v[t] = 0.0f;
  for (int c0 = 0; c0 < n; c0 += 4) {
    float tmp[4][T];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + i < n ? c0 + i : n - 1;  // in-range address; extra values are not added
#pragma unroll
      for (int t = 0; t < T; ++t) tmp[i][t] = ld_coh(base + ((size_t)c * T + t) * 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c0 + i < n)
#pragma unroll
        for (int t = 0; t < T; ++t) v[t] += tmp[i][t];
  }
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
      xn[t] = ld_coh(xp) + v0[t];
      st_coh(xp, xn[t]);
    }
    const int ss_idx = d.ph == 1 ? 2 * l + 1 : 2 * l + 2;
    float* ss = a.ss + ((size_t)ss_idx * (a.H / 64) + tau) * 16;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s2 = wave_sum(xn[t] * xn[t]);
      if (lane == 0) st_coh(ss + t, s2);
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

// Issues the loads of the first weight unit of wave w's stretch of phase d
// (weights do not depend on activations, so this can precede the barrier
// that makes the activations ready).  Returns false if the stretch is empty.
__device__ __forceinline__ bool prefetch_first(const StepArgs& a, const PhaseDesc& d, int w, int lane, Unit& out) {
  const int nsb = d.K / 256;
  Split sp;
  sp.Gw = d.gdn_jobs * kGdnJobWeight;
  sp.S = sp.Gw + (long)(d.N / 64) * d.nm * nsb;
  sp.W = a.wp[d.plan];
  if (w >= sp.W) return false;
  const long s0 = split_start(sp, w), s1 = split_start(sp, w + 1);
  if (s0 < sp.Gw) return false;  // this wave starts with Gated DeltaNet jobs
  const long u = s0 - sp.Gw, u1 = (s1 > sp.Gw ? s1 : sp.Gw) - sp.Gw;
  if (u >= u1) return false;
  const int tm = (int)(u / nsb), b0 = (int)(u % nsb);
  load_unit(d.W[tm % d.nm] + ((size_t)(tm / d.nm) * nsb + b0) * kUnitBytes, lane, out);
  return true;
}

// One segment of a wave's stretch: the units of one (tile, matrix) from u on;
// flushes the partial, takes the tile's ticket and, if last, runs the
// epilogue.  Returns the number of units done.  With USE_PRE, `pre` holds the
// segment's first unit.
template <int T, bool USE_PRE>
__device__ __forceinline__ int gemv_segment(const StepArgs& a, const PhaseDesc& d, const Split& sp, const QAct& act,
                                            long u, long u1, int w, int lane, unsigned* tickets, Unit& pre) {
  const int nsb = d.K / 256;
  const int tm = (int)(u / nsb);
  const int b0 = (int)(u % nsb);
  const int len = (int)((u1 - u) < (long)(nsb - b0) ? (u1 - u) : (long)(nsb - b0));
  const int tau = tm / d.nm, m = tm % d.nm;
  float acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = 0.0f;
  if (USE_PRE)
    dot4_range_from<T>(d.W[m] + (size_t)tau * nsb * kUnitBytes, b0, b0 + len, act, lane, acc, pre);
  else
    dot4_range<T>(d.W[m] + (size_t)tau * nsb * kUnitBytes, b0, b0 + len, act, lane, acc);
  const int lo = wave_of_weight(sp, sp.Gw + (long)tm * nsb);
  float* dst = a.part + ((size_t)tm * a.cmax[d.plan] + (w - lo)) * T * 64;
#pragma unroll
  for (int t = 0; t < T; ++t) st_coh(dst + t * 64 + lane, acc[t]);
  // ticket: the last contribution to this tile runs its epilogue
  int expect = 0;
  for (int mm = 0; mm < d.nm; ++mm) {
    const long uu = ((long)tau * d.nm + mm) * nsb;
    expect += wave_of_weight(sp, sp.Gw + uu + nsb - 1) - wave_of_weight(sp, sp.Gw + uu) + 1;
  }
  unsigned prev = 0;
  if (lane == 0) prev = ticket_add(tickets + (size_t)tau * kTicketStride);
  prev = uniform((int)__shfl(prev, 0, 64));
  if ((int)prev == expect - 1) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    epilogue<T>(a, d, sp, nsb, tau, lane);
  }
  return len;
}

template <int T, bool USE_PRE>
__device__ void gemv_units(const StepArgs& a, const PhaseDesc& d, const Split& sp, long s0, long s1, int w,
                           int lane, Unit& pre, bool have_pre) {
  QAct act;
  act.a8 = fresh(uniform(d.in.a8));
  act.ssg = fresh(uniform(d.in.ssg));
  act.K = d.K;
  act.T = T;
  long u = (s0 > sp.Gw ? s0 : sp.Gw) - sp.Gw;
  const long u1 = (s1 > sp.Gw ? s1 : sp.Gw) - sp.Gw;
  unsigned* tickets = a.tickets + ((size_t)d.layer * 4 + d.ph) * kTicketTiles * kTicketStride;
  if (USE_PRE && have_pre && u < u1) u += gemv_segment<T, true>(a, d, sp, act, u, u1, w, lane, tickets, pre);
  while (u < u1) u += gemv_segment<T, false>(a, d, sp, act, u, u1, w, lane, tickets, pre);
}

template <int T>
__device__ void gemv_phase(const StepArgs& a, const PhaseDesc& d, int w, int lane, Unit& pre, bool have_pre) {
  const int nsb = d.K / 256;
  Split sp;
  sp.Gw = d.gdn_jobs * kGdnJobWeight;
  sp.S = sp.Gw + (long)(d.N / 64) * d.nm * nsb;
  sp.W = a.wp[d.plan];
  if (w >= sp.W) return;
  const long s0 = split_start(sp, w), s1 = split_start(sp, w + 1);
  if (s0 < sp.Gw) {
    // Gated DeltaNet jobs whose start falls in this stretch; no unit was
    // prefetched for such a wave (see prefetch_first)
    for (long j = (s0 + kGdnJobWeight - 1) / kGdnJobWeight; j * kGdnJobWeight < s1 && j < d.gdn_jobs; ++j)
      gdn_job(a, d.layer, j, lane);
    gemv_units<T, false>(a, d, sp, s0, s1, w, lane, pre, false);
  } else {
    gemv_units<T, true>(a, d, sp, s0, s1, w, lane, pre, have_pre);
  }
}

// ------------------------------------------------------------ small phases
template <int T>
__device__ void prep_phase(const StepArgs& a, int w, int lane, int nw) {
  const int ntH = a.H / 64;
  for (int tau = w; tau < ntH; tau += nw) {
    float xv[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xv[t] = ld_coh(a.x + (size_t)t * a.H + tau * 64 + lane);
    float* ss = a.ss + (size_t)tau * 16;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float s2 = wave_sum(xv[t] * xv[t]);
      if (lane == 0) st_coh(ss + t, s2);
    }
    store_q8<T>(act_ref(a, 0, K_X, a.H), tau, lane, xv);
  }
}

__device__ void lm_prep_phase(const StepArgs& a, int w, int lane, int nw) {
  const int nc = a.H / 64;
  const int t = lane & 15, kq = lane >> 4;
  const float rl = rnorm_lane(a, 2 * a.L, lane);
  const float r = __shfl(rl, t, 64);
  const int tt = t < a.T ? t : 0;  // every lane loads an in-range value
  for (int c = w; c < nc; c += nw) {
    float* o = (float*)(a.frag + ((size_t)c * 64 + lane) * 32);
    float xr[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) xr[e] = ld_coh(a.x + (size_t)tt * a.H + 64 * c + 16 * kq + e);
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float x0 = t < a.T ? r * xr[e] : 0.0f, x1 = t < a.T ? r * xr[e + 1] : 0.0f;
      const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
      const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
      st_coh(o + e / 2, __builtin_bit_cast(float, (h2){h0, h1}));
      st_coh(o + 8 + e / 2, __builtin_bit_cast(float, (h2){l0, l1}));
    }
  }
}

// One 64-wide hidden chunk of 64 vocabulary rows: the weight fragments of
// the 4 row groups and the hi/lo fragments of the hidden rows.
struct LmChunk {
  u32x4 wa[4][2];
  u32x4 bh0, bh1, bl0, bl1;
};

__device__ __forceinline__ void lm_load(const StepArgs& a, int v0, int c, int l, int vl, int kq, LmChunk& x) {
  const u32x4* fp = (const u32x4*)(a.frag + ((size_t)c * 64 + l) * 32);
  x.bh0 = fp[0];
  x.bh1 = fp[1];
  x.bl0 = fp[2];
  x.bl1 = fp[3];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int v = v0 + 16 * g + vl;
    const int vv = v < a.V ? v : a.V - 1;  // in-range row; results of rows >= V are never used
    const u32x4* wpp = (const u32x4*)(a.lm + (size_t)vv * a.H + 64 * c + 16 * kq);
    x.wa[g][0] = __builtin_nontemporal_load(wpp);
    x.wa[g][1] = __builtin_nontemporal_load(wpp + 1);
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

__device__ __forceinline__ bool lm_better(float va, int ia, float vb, int ib) {
  if (ia < 0) return false;
  if (ib < 0) return true;
  if (va != va) return false;
  if (vb != vb) return true;
  return va > vb || (va == vb && ia < ib);
}

__device__ void lm_phase(const StepArgs& a) {
  constexpr int NW = kWavesPerBlock, TPT = kBlock / 16, RPP = 64 / TPT;  // threads per row t, rows per thread
  __shared__ float red[NW][64][16];
  __shared__ int last;
  __shared__ int fin[16];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
  const int vl = l & 15, kq = l >> 4;
  const int nc = a.H / 64;
  const int c0 = (nc * w) / NW, c1 = (nc * (w + 1)) / NW;
  const int nblk = (a.V + 63) / 64;
  const int t_own = threadIdx.x / TPT, part = threadIdx.x % TPT;
  float best = 0.0f;
  int bidx = -1;
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int v0 = blk * 64;
    f32x4 acc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[g] = (f32x4){0.f, 0.f, 0.f, 0.f};
    LmChunk b0c, b1c;  // ping-pong: the next chunk's loads are issued before this chunk's MFMAs
    if (c0 < c1) lm_load(a, v0, c0, l, vl, kq, b0c);
    for (int c = c0; c < c1; c += 2) {
      if (c + 1 < c1) lm_load(a, v0, c + 1, l, vl, kq, b1c);
      lm_mfma(b0c, acc);
      if (c + 1 >= c1) break;
      if (c + 2 < c1) lm_load(a, v0, c + 2, l, vl, kq, b0c);
      lm_mfma(b1c, acc);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w][16 * g + 4 * kq + i][vl] = acc[g][i];
    __syncthreads();
    for (int r = RPP * part; r < RPP * part + RPP; ++r) {
      const int v = v0 + r;
      if (v >= a.V) break;
      float xv = red[0][r][t_own];
#pragma unroll
      for (int q = 1; q < NW; ++q) xv += red[q][r][t_own];
      if (lm_better(xv, v, best, bidx)) {
        best = xv;
        bidx = v;
      }
    }
    __syncthreads();
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
  if (part == 0) {
    st_coh(a.lm_val + (size_t)blockIdx.x * 16 + t_own, best);
    st_coh((float*)a.lm_idx + (size_t)blockIdx.x * 16 + t_own, __builtin_bit_cast(float, bidx));
  }
  __syncthreads();
  if (threadIdx.x == 0) last = (ticket_add(a.lm_ticket) == gridDim.x - 1);
  __syncthreads();
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  best = 0.0f;
  bidx = -1;
  for (int b = part; b < (int)gridDim.x; b += TPT) {
    const float xv = ld_coh(a.lm_val + (size_t)b * 16 + t_own);
    const int iv = ld_coh_i(a.lm_idx + (size_t)b * 16 + t_own);
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
  if (blockIdx.x == 0 && threadIdx.x == 0) a.stamps[0] = wall_clock64();
  // the first weight unit of each phase is requested before the barrier that
  // precedes the phase
  Unit pre;
  bool have = prefetch_first(a, phase_desc(a, 0, 0), w, lane, pre);
  prep_phase<T>(a, w, lane, nw);
  grid_barrier(a, gen);
  for (int l = 0; l < a.L; ++l) {
    for (int ph = 0; ph < 4; ++ph) {
      const PhaseDesc d = phase_desc(a, ph, l);
      gemv_phase<T>(a, d, w, lane, pre, have);
      const int nph = ph == 3 ? 0 : ph + 1, nl = ph == 3 ? l + 1 : l;
      have = nl < a.L ? prefetch_first(a, phase_desc(a, nph, nl), w, lane, pre) : false;
      grid_barrier(a, gen);
    }
  }
  lm_prep_phase(a, w, lane, nw);
  grid_barrier(a, gen);
  lm_phase(a);
  if (blockIdx.x == 0 && threadIdx.x == 0) a.stamps[kMaxStamps - 1] = wall_clock64();
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
  hipEvent_t ev[2] = {nullptr, nullptr};  // around the last launch (no device memory)
  float last_ms = -1.0f;
};

namespace {

size_t a256(size_t n) { return (n + 255) / 256 * 256; }

struct StepLayout {
  int grid, waves;
  int wp[5], cmax[5];
  size_t off_ctrl, n_ctrl;  // zeroed before each launch: barrier, tickets
  size_t off_out, off_stamps, off_tickets, off_lmticket, off_table, off_a8, off_ssg, off_ss, off_part, off_frag, off_lmv,
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
  o += a256((size_t)d.n_layers * 4 * kTicketTiles * kTicketStride * 4);
  y.n_ctrl = o - y.off_ctrl;
  y.off_out = o;
  o += 256;
  y.off_stamps = o;
  o += a256(sizeof(uint64_t) * kMaxStamps);
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
  if (hipEventCreate(&st->ev[0]) != hipSuccess || hipEventCreate(&st->ev[1]) != hipSuccess) {
    st->ev[0] = st->ev[1] = nullptr;
  }
  *out = st;
  return MK_OK;
}

void mk_stack_destroy(mk_stack* st) {
  if (!st) return;
  for (int i = 0; i < 2; ++i)
    if (st->ev[i]) hipEventDestroy(st->ev[i]);
  delete st;
}

float mk_decode_step_last_ms(const mk_stack* st) { return st ? st->last_ms : -1.0f; }

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
  a.stamps = (uint64_t*)(w8 + y.off_stamps);
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
  if (st->ev[0]) hipEventRecord(st->ev[0], s);
  hipError_t e = hipLaunchCooperativeKernel((const void*)step_kernel(T), dim3(y.grid), dim3(kBlock), args, 0, s);
  if (st->ev[1]) hipEventRecord(st->ev[1], s);
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
  st->last_ms = -1.0f;
  if (st->ev[0] && st->ev[1]) hipEventElapsedTime(&st->last_ms, st->ev[0], st->ev[1]);
  if (hout[0]) return sfail(MK_ERR_DEVICE, "decode: grid-barrier watchdog fired");
  for (int g = 0; g < G; ++g) h_n_acc[g] = hout[16 + g];
  for (int t = 0; t < T; ++t) h_tokens[t] = hout[32 + t];
  set_error(MK_OK, "");
  return MK_OK;
}

int mk_decode_step_stamps(const mk_stack* st, int32_t T, const void* ws, uint64_t* h_stamps, int32_t n,
                          int64_t* h_clock_hz) {
  if (!st || !ws || !h_stamps || n < 1) return sfail(MK_ERR_ARG, "stamps: null argument");
  const StepLayout y = layout(st, T);
  const int m = n < kMaxStamps ? n : kMaxStamps;
  if (hipMemcpy(h_stamps, (const uint8_t*)ws + y.off_stamps, sizeof(uint64_t) * m, hipMemcpyDeviceToHost) !=
      hipSuccess)
    return sfail(MK_ERR_LAUNCH, "stamps: copy failed");
  if (h_clock_hz) {
    int dev = 0, khz = 0;
    hipGetDevice(&dev);
    hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    *h_clock_hz = (int64_t)khz * 1000;
  }
  return m;
}

}  // extern "C"
