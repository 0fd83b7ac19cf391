// The penalty of one logit whose token occurs c >= 1 times in the row's
// history: repeat (divide a positive logit, multiply a non-positive one),
// then frequency (c times), then presence, in fp32 with one rounding per
// operation, in that order (the library is built without floating-point
// contraction and with a correctly rounded divide).  "Speculative decoding
// on RDNA", section 04; the formulas are the reading the library takes.
#pragma once

#include "vs_internal.h"

namespace {

__device__ __forceinline__ float penalize_one(float l, int c, float rep, float pres, float freq) {
  const float l1 = (l > 0.f) ? (l / rep) : (l * rep);
  const float cf = static_cast<float>(c) * freq;
  const float l2 = l1 - cf;
  return l2 - pres;
}

}  // namespace
