// Wavefront-level helpers for the sampling kernels (one 64-lane wave per row
// or per window).  Sums that define a result run sequentially in lane order
// (every lane walks the same sequence through shuffles), which fixes the
// rounding order independently of the hardware's reduction trees.
#pragma once

#include "vs_internal.h"

namespace vs {

// Value of lane `src` (uniform across the wave) in every lane.  A lane read
// into a scalar register: no LDS round trip, so sequential loops over the
// lanes stay short.
__device__ __forceinline__ double bcast(double v, int src) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b & 0xffffffffu), src));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b >> 32), src));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ int bcast(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

// Sequential sum of w over lanes [0, n), lane order, fp64.  Lanes holding
// zero are skipped: the sum starts at +0 and adding a zero of either sign to
// it never changes it (it cannot become -0), so the result is the same as
// adding every lane.
__device__ __forceinline__ double seq_sum(double w, int n) {
  const int lane = threadIdx.x & 63;
  uint64_t m = __ballot(lane < n && w != 0.0);
  double s = 0.0;
  while (m) {
    s += bcast(w, __ffsll(static_cast<long long>(m)) - 1);
    m &= m - 1;
  }
  return s;
}

// Makes this wave's LDS writes visible to its other lanes before they read.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Inverse-CDF draw over lanes [0, n): the first lane j with u * C_n < C_j,
// C_j the sequential fp64 sum of w over lanes 0..j.  If rounding leaves no
// such lane, the last lane with positive weight (else 0).  run: this wave's
// 64 LDS slots, where lane 0 records each C_j for lane j to read back.
// Zero lanes are skipped as in seq_sum; one is never the first lane to pass
// (C_j equals the previous lane's sum, which then passes first, or 0).
__device__ __forceinline__ int seq_draw(double w, int n, float u, double* run) {
  const int lane = threadIdx.x & 63;
  const bool live = lane < n && w != 0.0;
  uint64_t m = __ballot(live);
  wave_lds_sync();  // a previous use of the slots has been read
  double acc = 0.0;
  while (m) {
    const int j = __ffsll(static_cast<long long>(m)) - 1;
    acc += bcast(w, j);
    if (lane == 0) run[j] = acc;
    m &= m - 1;
  }
  wave_lds_sync();
  const double mine = live ? run[lane] : 0.0;
  const double target = static_cast<double>(u) * acc;
  const uint64_t hit = __ballot(lane < n && target < mine);
  if (hit) return __ffsll(static_cast<long long>(hit)) - 1;
  const uint64_t pos = __ballot(lane < n && w > 0.0);
  return pos ? 63 - __clzll(static_cast<long long>(pos)) : 0;
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = lane == 0 ? 0ull : (mask & (~0ull >> (64 - lane)));
  return __popcll(below);
}

}  // namespace vs
