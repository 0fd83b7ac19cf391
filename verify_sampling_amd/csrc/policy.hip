// sample_policy_rows: the sampler distribution of each row (+ optional draw).
//
// "Speculative decoding on RDNA", §03 "how hipfire does it": temperature,
// then top-k (absent -> 20, 0 -> the 64-wide pool), then min-p, then top-p,
// with the same pool, tie order and summation for p (target rows) and q (the
// draft's re-scored candidates).
//
// One 64-lane wave per row, one candidate per lane.  The candidates are
// bitonic-sorted into pool order by their 64-bit order key (skipped when
// they already are in that order, as topk_rows leaves them); the weights
// exp((l_j - l_0)/T) are computed lane-parallel in fp64.  Every sum the
// result depends on is taken sequentially in pool order, so the
// distribution does not depend on the hardware's reduction order.  Both
// filters compare ratios of weights and are evaluated on the unnormalised
// weights; the kept weights are normalised once and rounded to fp32.
//
// One sequential prefix scan over the min-p survivors' weights (the other
// candidates would add +0.0 to a non-negative sum, which changes nothing, so
// they are skipped) gives every sum
// the policy needs: its total is the top-p reference sum, the exclusive
// prefix at a candidate is the mass kept before it (the scan is
// non-decreasing, so the top-p survivors are the min-p survivors up to the
// first failure, plus always the first one), and the inclusive prefix at
// the last top-p survivor is the normaliser.  Each of these equals the
// corresponding separate left-to-right sum bit for bit.

#include "policy_dev.h"

namespace {

constexpr int ROWS_PER_BLOCK = 4;

__global__ void __launch_bounds__(64 * ROWS_PER_BLOCK)
policy_kernel(const float* __restrict__ vals, const int32_t* __restrict__ ids, int64_t ld, int rows,
              int M, float temperature, int k_eff, float top_p, float min_p,
              int32_t* __restrict__ dist_ids, float* __restrict__ dist_probs,
              int32_t* __restrict__ dist_len, int64_t ld_dist, const float* __restrict__ u,
              int32_t* __restrict__ drawn) {
  // running sums of the sequential scans, one slot per candidate: lane 0
  // records each partial sum, every lane reads its own after the loop
  __shared__ double scan[ROWS_PER_BLOCK][64];
  const int wave = vs::wave_index();
  const int row = blockIdx.x * ROWS_PER_BLOCK + wave;
  if (row >= rows) return;  // whole wave; the kernel has no block-wide barriers
  policy_row(vals + static_cast<int64_t>(row) * ld, ids + static_cast<int64_t>(row) * ld, M, temperature,
             k_eff, top_p, min_p, dist_ids + static_cast<int64_t>(row) * ld_dist,
             dist_probs + static_cast<int64_t>(row) * ld_dist, dist_len + row,
             u != nullptr ? u + row : nullptr, drawn != nullptr ? drawn + row : nullptr, scan[wave]);
}

}  // namespace

extern "C" int sample_policy_rows(const float* vals, const int32_t* ids, int64_t ld, int rows, int M,
                                  float temperature, int top_k, float top_p, float min_p,
                                  int32_t* dist_ids, float* dist_probs, int32_t* dist_len,
                                  int64_t ld_dist, const float* u, int32_t* drawn,
                                  hipStream_t stream) {
  if (!vals || !ids || !dist_ids || !dist_probs || !dist_len) return VS_ERR_NULL;
  if ((u == nullptr) != (drawn == nullptr)) return VS_ERR_NULL;
  if (rows < 1 || M < 1 || M > VS_POOL || ld < M || ld_dist < M) return VS_ERR_SHAPE;
  if (__builtin_isnan(temperature) || __builtin_isnan(top_p) || __builtin_isnan(min_p))
    return VS_ERR_PARAM;
  if (__builtin_isinf(temperature)) return VS_ERR_PARAM;
  const int k_eff = policy_k_eff(top_k);
  const int blocks = (rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  policy_kernel<<<dim3(blocks), dim3(64 * ROWS_PER_BLOCK), 0, stream>>>(
      vals, ids, ld, rows, M, temperature, k_eff, top_p, min_p, dist_ids, dist_probs, dist_len,
      ld_dist, u, drawn);
  return vs::check_launch();
}
