// Internal helpers shared by the library's translation units (host and device).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "verify_sampling.h"

namespace vs {

// Records the HIP error text for vs_last_error_detail() and maps it to VS_ERR_HIP.
int hip_status(hipError_t e);

// Checks the launch that was just enqueued.
inline int check_launch() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? VS_OK : hip_status(e);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The wavefront's index within its workgroup (64-lane waves), marked uniform
// so that loops and addresses derived from it stay in scalar registers.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// ---------------------------------------------------------------- ordering keys
//
// The pool order (value descending, index ascending, NaN below -inf, -0 == +0)
// as one unsigned 64-bit key, larger = earlier:
//   high 32 bits: the value mapped to an unsigned int that increases with the
//                 value (every NaN maps to 0, -0 to the image of +0);
//   low 32 bits:  the bitwise complement of the index, so lower indices win.
// Indices are < 2^31, so every real element's key is > 0, and 0 can serve as
// a sentinel that ranks below every real element.
__device__ __forceinline__ uint32_t value_key(uint32_t bits) {
  if ((bits & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN
  if (bits == 0x80000000u) bits = 0u;                  // -0 -> +0
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

__device__ __forceinline__ uint64_t order_key(uint32_t bits, uint32_t index) {
  return (static_cast<uint64_t>(value_key(bits)) << 32) | static_cast<uint64_t>(~index);
}

__device__ __forceinline__ uint32_t key_index(uint64_t key) {
  return ~static_cast<uint32_t>(key & 0xffffffffull);
}

// Bitonic sort of one 64-bit key per lane across a 64-lane wavefront,
// descending (lane 0 ends with the largest key).  Keys travel with a 32-bit
// payload.
__device__ __forceinline__ void wave_sort_desc(uint64_t& key, uint32_t& payload) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      uint32_t lo = static_cast<uint32_t>(key), hi = static_cast<uint32_t>(key >> 32);
      uint32_t olo = __shfl_xor(lo, stride, 64), ohi = __shfl_xor(hi, stride, 64);
      uint32_t opay = __shfl_xor(payload, stride, 64);
      uint64_t other = (static_cast<uint64_t>(ohi) << 32) | olo;
      // Within each block of `size`, the lower half of the lanes of a
      // compare pair keeps the larger key when the block sorts descending.
      const bool lower = (lane & stride) == 0;
      const bool desc = (lane & size) == 0 || size == 64;
      const bool take_max = (lower == desc);
      const bool swap = take_max ? (other > key) : (other < key);
      if (swap) {
        key = other;
        payload = opay;
      }
    }
  }
}

}  // namespace vs
