// mk_gdn.hip — Gated DeltaNet decode step with rollback (page: richland.au
// single-stream article, "What shipped": the recurrent state is committed
// only through the surely-accepted token and drafts are replayed from a small
// (k, v, g, beta) ring; 48 of the 64 layers carry this constant-size state).
//
// Per head, S is dk x dv (S[i][j], i key index, j value index) and one row
// (q, k, v, g, beta) applies
//     u = S^T k;  S <- g S + beta k (v - g u)^T   (= g (I - beta k k^T) S + beta k v^T)
//     o = S^T q   (after the update).
// Layout of the work: one block of 128 threads per head, thread j owns
// column j of S in 128 registers, so S^T k and S^T q are per-thread dot
// products against the wave-uniform k and q (read through the scalar cache);
// S is read from HBM once and written once per step.
#include "mk_device.h"
#include "mk_internal.h"

namespace mk {

constexpr int kD = 128;
constexpr int kRingRow = 2 * kD + 2;  // k[128], v[128], g, beta

// Returns p unchanged, but only once `dep` has been computed, so loads
// through the result cannot be issued before that point.  Used to bound how
// far ahead the compiler requests the wave-uniform k and q chunks (hoisting
// all of them would need 256 scalar registers).
__device__ __forceinline__ const float* after(const float* p, float dep) {
  asm volatile("" : "+s"(p) : "v"(dep));
  return p;
}
// Same for a store base: the 128 per-element addresses of a column are then
// formed where they are used instead of being hoisted and kept live.
__device__ __forceinline__ float* after_w(float* p, float dep) {
  asm volatile("" : "+s"(p) : "v"(dep));
  return p;
}

// One row of the delta rule on the column this thread owns; k and q are
// wave-uniform and streamed 8 floats at a time through the scalar cache, two
// chunks ahead of their use.  Pass 1: u = S^T k.  Pass 2: S <- g S + k c with
// c = beta (v - g u), fused with o = S^T q on the updated column (WITH_Q).
template <bool WITH_Q>
__device__ __forceinline__ float gdn_row(float (&S)[kD], const float* kp, const float* qp, float vj, float g,
                                         float beta) {
  float u = 0.0f;
  f32x8 k0 = *as_const<f32x8>(kp), k1 = *as_const<f32x8>(kp + 8);
#pragma unroll
  for (int c = 0; c < kD / 8; ++c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) u = __builtin_fmaf(k0[e], S[8 * c + e], u);
    k0 = k1;
    if (c + 2 < kD / 8) k1 = *as_const<f32x8>(after(kp, u) + 8 * (c + 2));
  }
  const float cc = beta * (vj - g * u);
  float o = 0.0f;
  k0 = *as_const<f32x8>(after(kp, cc));
  k1 = *as_const<f32x8>(after(kp, cc) + 8);
  if constexpr (WITH_Q) {
    f32x8 q0 = *as_const<f32x8>(qp), q1 = *as_const<f32x8>(qp + 8);
#pragma unroll
    for (int c = 0; c < kD / 8; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        S[8 * c + e] = __builtin_fmaf(k0[e], cc, g * S[8 * c + e]);
        o = __builtin_fmaf(q0[e], S[8 * c + e], o);
      }
      k0 = k1;
      q0 = q1;
      if (c + 2 < kD / 8) {
        k1 = *as_const<f32x8>(after(kp, o) + 8 * (c + 2));
        q1 = *as_const<f32x8>(after(qp, o) + 8 * (c + 2));
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < kD / 8; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) S[8 * c + e] = __builtin_fmaf(k0[e], cc, g * S[8 * c + e]);
      k0 = k1;
      if (c + 2 < kD / 8) k1 = *as_const<f32x8>(after(kp, S[8 * c + 7]) + 8 * (c + 2));
    }
  }
  return o;
}

__device__ __forceinline__ int replay_count(const GdnArgs& a) {
  if (!a.n_acc) return 0;
  int n = *as_const<int32_t>(a.n_acc);
  return n < 0 ? 0 : (n > a.T_max - 1 ? a.T_max - 1 : n);
}

__device__ __forceinline__ void replay(const GdnArgs& a, int h, int nrep, int j, float (&S)[kD]) {
  const float* ring = a.ring + (size_t)h * (a.T_max - 1) * kRingRow;
  for (int r = 0; r < nrep; ++r) {
    const float* row = ring + (size_t)r * kRingRow;
    const float vj = row[kD + j];
    const float g = *as_const<float>(row + 2 * kD), beta = *as_const<float>(row + 2 * kD + 1);
    gdn_row<false>(S, row, nullptr, vj, g, beta);
  }
}

__global__ __launch_bounds__(128) void k_gdn_step(GdnArgs a) {
  const int h = blockIdx.x, j = threadIdx.x;
  float* Sh = a.S + (size_t)h * kD * kD;
  float S[kD];
#pragma unroll
  for (int i = 0; i < kD; ++i) S[i] = __builtin_nontemporal_load(Sh + (size_t)i * kD + j);
  replay(a, h, replay_count(a), j, S);
  __syncthreads();  // every wave has read the ring before it is overwritten
  float* ring = a.ring + (size_t)h * (a.T_max - 1) * kRingRow;
  {
    // row 0 (the token accepted last step) is committed right after its update
    const size_t th = h;
    const float g = *as_const<float>(a.g + th), beta = *as_const<float>(a.beta + th);
    const float o0 = gdn_row<true>(S, a.k + th * kD, a.q + th * kD, a.v[th * kD + j], g, beta);
    a.o[th * kD + j] = o0;
    float* Sw = after_w(Sh, o0) + j;
#pragma unroll
    for (int i = 0; i < kD; ++i) __builtin_nontemporal_store(S[i], Sw + (size_t)i * kD);
  }
  for (int t = 1; t < a.T; ++t) {
    const size_t th = (size_t)t * a.nh + h;
    const float vj = a.v[th * kD + j];
    const float g = *as_const<float>(a.g + th), beta = *as_const<float>(a.beta + th);
    a.o[th * kD + j] = gdn_row<true>(S, a.k + th * kD, a.q + th * kD, vj, g, beta);
    float* row = ring + (size_t)(t - 1) * kRingRow;
    row[j] = a.k[th * kD + j];  // thread j copies element j of k
    row[kD + j] = vj;
    // (g, beta) at row[2*kD], row[2*kD+1]: every thread stores the same pair
    // of values (no divergent branch inside the row loop)
    row[2 * kD + (j & 1)] = (j & 1) ? beta : g;
  }
}

__global__ __launch_bounds__(128) void k_gdn_commit(GdnArgs a) {
  const int h = blockIdx.x, j = threadIdx.x;
  const int nrep = replay_count(a);
  if (nrep == 0) return;
  float* Sh = a.S + (size_t)h * kD * kD;
  float S[kD];
#pragma unroll
  for (int i = 0; i < kD; ++i) S[i] = Sh[(size_t)i * kD + j];
  replay(a, h, nrep, j, S);
  float* Sw = after_w(Sh, S[kD - 1]) + j;
#pragma unroll
  for (int i = 0; i < kD; ++i) Sw[(size_t)i * kD] = S[i];
}

hipError_t launch_gdn_step(const GdnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_gdn_step, dim3(a.nh), dim3(kD), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gdn_commit(const GdnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_gdn_commit, dim3(a.nh), dim3(kD), 0, st, a);
  return hipGetLastError();
}

}  // namespace mk
