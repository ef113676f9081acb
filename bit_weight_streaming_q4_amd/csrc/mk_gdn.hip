// mk_gdn.hip — standalone Gated DeltaNet step / commit launches (the device
// code is in mk_gdn.h and is shared with the persistent decode step).
#include "mk_gdn.h"
#include "mk_internal.h"

namespace mk {

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
  // 128-B chunks of k and q (two 64-B scalar loads each): a quarter of the
  // dependent scalar loads per row pass of 32-B chunks
  gdn_half_step<32>(x, lane);
}

__global__ __launch_bounds__(64) void k_gdn_commit(GdnArgs a) {
  const int h = blockIdx.x, half = blockIdx.y, lane = threadIdx.x;
  const int par = *as_const<int32_t>(a.n_acc + 1) & 1;
  const float* rd = a.ring + ((size_t)par * a.nh + h) * (a.T_max - 1) * kRingRow;
  gdn_half_commit<32>(a.S + (size_t)h * kD * kD, rd, checked_acc(a.n_acc, a.T_max, h == 0 && half == 0 && lane == 0),
                  half, lane);
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
