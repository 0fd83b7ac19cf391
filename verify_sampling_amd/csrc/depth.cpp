// vs_choose_depth: the draft depth of the next verify window.
//
// "Speculative decoding on RDNA", §05 "What a verify row costs on RDNA": a
// window of R rows has a measured cost; the depth is chosen per window as
// the k that maximises the expected emitted tokens, 1 plus the running
// products of the per-depth acceptance rates, per unit of window cost, with
// one token per plain decode step (k = 0) as the fallback.  Host code: the
// inputs are a handful of numbers per window.

#include <cmath>

#include "verify_sampling.h"

extern "C" int vs_choose_depth(const double* alpha, int kmax, const double* cost, double* rate) {
  if (!cost || (kmax > 0 && !alpha)) return VS_ERR_NULL;
  if (kmax < 0 || kmax > VS_MAX_DRAFTS) return VS_ERR_SHAPE;
  for (int k = 0; k <= kmax; ++k)
    if (!(cost[k] > 0.0) || !std::isfinite(cost[k])) return VS_ERR_PARAM;
  for (int j = 0; j < kmax; ++j)
    if (!(alpha[j] >= 0.0 && alpha[j] <= 1.0)) return VS_ERR_PARAM;
  // E(k) = 1 + sum_{j<=k} prod_{i<=j} alpha[i-1], accumulated in increasing j
  double total = 1.0, run = 1.0;
  int best = 0;
  double best_rate = total / cost[0];
  for (int k = 1; k <= kmax; ++k) {
    run = run * alpha[k - 1];
    total = total + run;
    const double r = total / cost[k];
    if (r > best_rate) {  // ties keep the smaller depth
      best = k;
      best_rate = r;
    }
  }
  if (rate) *rate = best_rate;
  return best;
}
