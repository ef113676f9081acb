// mk_gdn.hip — standalone Gated DeltaNet step / commit launches (the device
// code is in mk_gdn.h and is shared with the persistent decode step).
#include "mk_gdn.h"
#include "mk_internal.h"

namespace mk {

// Touches, one dword per 128-B line, the inputs this half-head wave reads row
// by row: nrep replayed ring rows (k, v, g, beta: 258 floats each, from rd)
// and T new rows (k and q of the head, v of this half).  Issued before the
// state's loads, the lines reach L2 while the state streams in; otherwise
// each row's chains of dependent k and q loads would each wait on HBM.
// Returns the OR of what was read, which the caller keeps live to the end
// (no wait is then placed before the state's loads).
__device__ __forceinline__ uint32_t touch_rows(const float* rd, int nrep, const float* k, const float* q,
                                               const float* v, size_t sqk, size_t sv, int T, int half, int lane) {
  constexpr int kRingLines = (kRingRow * 4 + 127) / 128;  // 9
  const int nnew = 10 * T, nall = nnew + kRingLines * nrep;
  uint32_t acc = 0;
  for (int id = lane; id < nall; id += 64) {
    const float* p;
    if (id < nnew) {
      const int t = id / 10, w = id - 10 * t;
      p = w < 4 ? k + t * sqk + 32 * w : w < 8 ? q + t * sqk + 32 * (w - 4) : v + t * sv + 64 * half + 32 * (w - 8);
    } else {
      const int r = (id - nnew) / kRingLines, w = id - nnew - kRingLines * r;
      p = rd + (size_t)r * kRingRow + min(32 * w, kRingRow - 1);
    }
    acc |= *(const uint32_t*)p;
  }
  return acc;
}

// grid (nh, 2): block = one wave = half a head.
__global__ __launch_bounds__(64) void k_gdn_step(GdnArgs a) {
  const int h = blockIdx.x, half = blockIdx.y, lane = threadIdx.x;
  const int par = *as_const<int32_t>(a.n_acc + 1) & 1;
  GdnHalf x;
  x.S = a.S + (size_t)h * kD * kD;
  x.ring_rd = a.ring + ((size_t)par * a.nh + h) * (a.T_max - 1) * kRingRow;
  x.ring_wr = a.ring + ((size_t)(par ^ 1) * a.nh + h) * (a.T_max - 1) * kRingRow;
  x.nrep = a.use_prev ? checked_acc(a.n_acc, a.T_max, h == 0 && half == 0 && lane == 0) : 0;
  x.q = a.q + (size_t)h * kD;
  x.k = a.k + (size_t)h * kD;
  x.v = a.v + (size_t)h * kD;
  x.g = a.g + h;
  x.beta = a.beta + h;
  x.sqk = (size_t)a.nh * kD;
  x.sv = (size_t)a.nh * kD;
  x.sgb = a.nh;
  x.o = a.o + (size_t)h * kD;
  x.so = (size_t)a.nh * kD;
  x.T = a.T;
  x.half = half;
  const uint32_t warm = touch_rows(x.ring_rd, x.nrep, x.k, x.q, x.v, x.sqk, x.sv, x.T,
                                   half, lane);
  // 128-B chunks of k and q (two 64-B scalar loads each): a quarter of the
  // dependent scalar loads per row pass of 32-B chunks
  gdn_half_step<32>(x, lane);
  asm volatile("" ::"v"(warm));
}

__global__ __launch_bounds__(64) void k_gdn_commit(GdnArgs a) {
  const int h = blockIdx.x, half = blockIdx.y, lane = threadIdx.x;
  const int par = *as_const<int32_t>(a.n_acc + 1) & 1;
  const float* rd = a.ring + ((size_t)par * a.nh + h) * (a.T_max - 1) * kRingRow;
  const int nrep = checked_acc(a.n_acc, a.T_max, h == 0 && half == 0 && lane == 0);
  const uint32_t warm = touch_rows(rd, nrep, nullptr, nullptr, nullptr, 0, 0, 0, half, lane);
  gdn_half_commit<32>(a.S + (size_t)h * kD * kD, rd, nrep, half, lane);
  asm volatile("" ::"v"(warm));
}

// After a step: its rows are in the other ring half.
__global__ void k_gdn_flip(int32_t* n_acc) { n_acc[1] ^= 1; }
// After a commit: nothing left to replay.
__global__ void k_gdn_clear(int32_t* n_acc) { n_acc[0] = 0; }

hipError_t launch_gdn_step(const GdnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_gdn_step, dim3(a.nh, 2), dim3(64), 0, st, a);
  hipLaunchKernelGGL(k_gdn_flip, dim3(1), dim3(1), 0, st, a.n_acc);
  return hipGetLastError();
}

hipError_t launch_gdn_commit(const GdnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_gdn_commit, dim3(a.nh, 2), dim3(64), 0, st, a);
  hipLaunchKernelGGL(k_gdn_clear, dim3(1), dim3(1), 0, st, a.n_acc);
  return hipGetLastError();
}

}  // namespace mk
