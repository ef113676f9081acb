// mk_gdn.h — device code of the Gated DeltaNet decode step with rollback
// (page: richland.au single-stream article, "What shipped": the recurrent
// state is committed only through the surely-accepted token and drafts are
// replayed from a small (k, v, g, beta) ring).
//
// Per head, S is dk x dv = 128 x 128 (S[i][j], i key index, j value index);
// one row (q, k, v, g, beta) applies
//     u = S^T k;  S <- g S + beta k (v - g u)^T   (= g (I - beta k k^T) S + beta k v^T)
//     o = S^T q   (after the update).
// Work unit: one wave = half a head (64 value columns, lane = column j).
// Each lane keeps its column of S in 128 registers, so S^T k and S^T q are
// per-lane dot products against the wave-uniform k and q, which are read
// through the scalar cache.  The two halves of a head share nothing but the
// ring's (k, g, beta), which is double-buffered by step parity, so they
// never wait for each other.  S is read once and written once per step.
#pragma once
#include "mk_device.h"

namespace mk {

constexpr int kD = 128;
constexpr int kRingRow = 2 * kD + 2;  // k[128], v[128], g, beta

// Returns p unchanged, but only once `dep` has been computed, so loads
// through the result cannot be issued before that point.  Bounds how far
// ahead the compiler requests the wave-uniform k and q chunks (requesting
// all of them would need 256 scalar registers).
__device__ __forceinline__ const float* after(const float* p, float dep) {
  asm volatile("" : "+s"(p) : "v"(dep));
  return p;
}
// Same for a store base: per-element addresses are formed where they are
// used instead of being hoisted and kept live.
__device__ __forceinline__ float* after_w(float* p, float dep) {
  asm volatile("" : "+s"(p) : "v"(dep));
  return p;
}

// One row of the delta rule on the column this lane owns; k and q are
// streamed CH floats at a time (one scalar load each), two chunks ahead of
// their use.  Pass 1: u = S^T k.  Pass 2: S <- g S + k c with
// c = beta (v - g u), fused with o = S^T q on the updated column when WITH_Q.
// The arithmetic and its order do not depend on CH.
template <bool WITH_Q, int CH = 8>
__device__ __forceinline__ float gdn_row(float (&S)[kD], const float* kp, const float* qp, float vj, float g,
                                         float beta) {
  typedef float vec __attribute__((ext_vector_type(CH)));
  constexpr int NC = kD / CH;
  kp = uniform(kp);
  if constexpr (WITH_Q) qp = uniform(qp);
  float u = 0.0f;
  vec k0 = *as_const<vec>(kp), k1 = *as_const<vec>(kp + CH);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int e = 0; e < CH; ++e) u = __builtin_fmaf(k0[e], S[CH * c + e], u);
    k0 = k1;
    if (c + 2 < NC) k1 = *as_const<vec>(after(kp, u) + CH * (c + 2));
  }
  const float cc = beta * (vj - g * u);
  float o = 0.0f;
  k0 = *as_const<vec>(after(kp, cc));
  k1 = *as_const<vec>(after(kp, cc) + CH);
  if constexpr (WITH_Q) {
    vec q0 = *as_const<vec>(qp), q1 = *as_const<vec>(qp + CH);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int e = 0; e < CH; ++e) {
        S[CH * c + e] = __builtin_fmaf(k0[e], cc, g * S[CH * c + e]);
        o = __builtin_fmaf(q0[e], S[CH * c + e], o);
      }
      k0 = k1;
      q0 = q1;
      if (c + 2 < NC) {
        k1 = *as_const<vec>(after(kp, o) + CH * (c + 2));
        q1 = *as_const<vec>(after(qp, o) + CH * (c + 2));
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int e = 0; e < CH; ++e) S[CH * c + e] = __builtin_fmaf(k0[e], cc, g * S[CH * c + e]);
      k0 = k1;
      if (c + 2 < NC) k1 = *as_const<vec>(after(kp, S[CH * c + CH - 1]) + CH * (c + 2));
    }
  }
  return o;
}

// One half-head step.  Row t of the inputs is at q + t*sqk, k + t*sqk,
// v + t*sv, g + t*sgb, beta + t*sgb; output row t at o + t*so.
struct GdnHalf {
  float* S;              // this head's state [128][128]
  const float* ring_rd;  // this head's ring half holding the previous step's rows
  float* ring_wr;        // this head's ring half receiving this step's rows 1..T-1
  int nrep;              // previous-step rows to replay (accept length)
  const float *q, *k, *v, *g, *beta;
  size_t sqk, sv, sgb;
  float* o;
  size_t so;
  int T, half;
};

template <int CH = 8>
__device__ __forceinline__ void gdn_half_step(const GdnHalf& a, int lane) {
  const int j = 64 * a.half + lane;
  float S[kD];
  {
    const float* Sr = a.S + j;
#pragma unroll
    for (int i = 0; i < kD; ++i) S[i] = __builtin_nontemporal_load(Sr + (size_t)i * kD);
  }
  for (int r = 0; r < a.nrep; ++r) {
    const float* row = a.ring_rd + (size_t)r * kRingRow;
    const float vj = row[kD + j];
    const float g = *as_const<float>(row + 2 * kD), beta = *as_const<float>(row + 2 * kD + 1);
    gdn_row<false, CH>(S, row, nullptr, vj, g, beta);
  }
  {
    // row 0 (the token accepted on the previous step) is committed right away
    const float g = *as_const<float>(a.g), beta = *as_const<float>(a.beta);
    const float o0 = gdn_row<true, CH>(S, a.k, a.q, a.v[j], g, beta);
    a.o[j] = o0;
    float* Sw = after_w(uniform(a.S), o0) + j;
#pragma unroll
    for (int i = 0; i < kD; ++i) __builtin_nontemporal_store(S[i], Sw + (size_t)i * kD);
  }
  for (int t = 1; t < a.T; ++t) {
    const float* kt = a.k + t * a.sqk;
    const float vj = a.v[t * a.sv + j];
    const float g = *as_const<float>(a.g + t * a.sgb), beta = *as_const<float>(a.beta + t * a.sgb);
    a.o[t * a.so + j] = gdn_row<true, CH>(S, kt, a.q + t * a.sqk, vj, g, beta);
    float* row = a.ring_wr + (size_t)(t - 1) * kRingRow;
    row[j] = kt[j];
    row[kD + j] = vj;
    // (g, beta): every lane of half 0 stores the same pair (no divergent branch)
    if (a.half == 0) row[2 * kD + (lane & 1)] = (lane & 1) ? beta : g;
  }
}

// Replays ring rows into the committed state (no new rows).
template <int CH = 8>
__device__ __forceinline__ void gdn_half_commit(float* Sh, const float* ring_rd, int nrep, int half, int lane) {
  if (nrep <= 0) return;
  const int j = 64 * half + lane;
  float S[kD];
#pragma unroll
  for (int i = 0; i < kD; ++i) S[i] = Sh[(size_t)i * kD + j];
  for (int r = 0; r < nrep; ++r) {
    const float* row = ring_rd + (size_t)r * kRingRow;
    const float vj = row[kD + j];
    const float g = *as_const<float>(row + 2 * kD), beta = *as_const<float>(row + 2 * kD + 1);
    gdn_row<false, CH>(S, row, nullptr, vj, g, beta);
  }
  float* Sw = after_w(uniform(Sh), S[kD - 1]) + j;
#pragma unroll
  for (int i = 0; i < kD; ++i) Sw[(size_t)i * kD] = S[i];
}

// The accept length n_acc[0] to replay: 0..T_max-1.  A value outside that
// range replays nothing, and `report` (one lane of the launch) sets the
// state's status word n_acc[2].
__device__ __forceinline__ int checked_acc(int32_t* n_acc, int T_max, bool report) {
  const int n = *as_const<int32_t>(n_acc);
  if (n >= 0 && n < T_max) return n;
  if (report) n_acc[2] = 1;
  return 0;
}

}  // namespace mk
