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

#include "wave_ops.h"

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
  const int lane = threadIdx.x & 63;
  const int wave = vs::wave_index();
  const int row = blockIdx.x * ROWS_PER_BLOCK + wave;
  if (row >= rows) return;  // whole wave; the kernel has no block-wide barriers
  double* run = scan[wave];

  const float* vrow = vals + static_cast<int64_t>(row) * ld;
  const int32_t* irow = ids + static_cast<int64_t>(row) * ld;
  uint64_t key = 0;
  uint32_t vbits = 0;
  if (lane < M) {
    vbits = __builtin_bit_cast(uint32_t, vrow[lane]);
    const int32_t id = irow[lane];
    if (id >= 0) key = vs::order_key(vbits, static_cast<uint32_t>(id));
  }
  // already in pool order (descending keys, empty slots last)?  Keys are
  // unique, so this holds exactly when no lane is below its successor.
  const uint32_t next_lo = __shfl_down(static_cast<uint32_t>(key), 1, 64);
  const uint32_t next_hi = __shfl_down(static_cast<uint32_t>(key >> 32), 1, 64);
  const uint64_t next = lane == 63 ? 0ull : ((static_cast<uint64_t>(next_hi) << 32) | next_lo);
  if (__ballot(key < next) != 0) vs::wave_sort_desc(key, vbits);  // lane j: the j-th candidate
  const bool real = key != 0;
  const int n_real = __popcll(__ballot(real));
  const int32_t tok = real ? static_cast<int32_t>(vs::key_index(key)) : -1;
  const float v = __builtin_bit_cast(float, vbits);

  bool keep = false;
  float prob = 0.f;
  if (n_real > 0) {
    bool one_hot = !(temperature > 0.f);
    double e = 0.0;
    if (!one_hot) {
      const float l0 = __builtin_bit_cast(float, vs::bcast(static_cast<int>(vbits), 0));
      const double T = static_cast<double>(temperature);
      const bool cand = real && lane < k_eff;
      if (__builtin_isinf(l0) && l0 > 0.f) {
        e = (cand && __builtin_isinf(v) && v > 0.f) ? 1.0 : 0.0;
      } else if (!__builtin_isfinite(l0)) {
        one_hot = true;
      } else {
        e = (cand && __builtin_isfinite(v))
                ? exp((static_cast<double>(v) - static_cast<double>(l0)) / T)
                : 0.0;
      }
    }
    if (!one_hot) {
      const double e0 = vs::bcast(e, 0);
      if (!(e0 > 0.0)) one_hot = true;
      if (!one_hot) {
        // weight-0 candidates carry no mass; min-p relative to the first
        const bool keep1 = e > 0.0 && e >= static_cast<double>(min_p) * e0;
        const double w1 = keep1 ? e : 0.0;
        // the scan runs over the min-p survivors only: lanes of weight 0 add
        // nothing and their prefixes are never used
        const uint64_t k1 = __ballot(keep1);
        double acc = 0.0;
        for (uint64_t m = k1; m; m &= m - 1) {
          const int j = __ffsll(static_cast<long long>(m)) - 1;
          if (lane == 0) run[j] = acc;
          acc += vs::bcast(w1, j);
        }
        vs::wave_lds_sync();
        const double excl = keep1 ? run[lane] : 0.0;
        const double incl = excl + w1;  // the scan's value after this lane, same rounding
        const double tp = static_cast<double>(top_p);
        bool keep2 = keep1;
        if (tp < 1.0) {
          const int first = k1 ? __ffsll(static_cast<long long>(k1)) - 1 : -1;
          keep2 = keep1 && (excl < tp * acc || lane == first);
        }
        const uint64_t k2 = __ballot(keep2);
        const double z = k2 ? vs::bcast(incl, 63 - __clzll(static_cast<long long>(k2))) : 1.0;
        keep = keep2;
        prob = keep ? static_cast<float>(e / z) : 0.f;
      }
    }
    if (one_hot) {
      keep = lane == 0;
      prob = keep ? 1.f : 0.f;
    }
  }

  const uint64_t kmask = __ballot(keep);
  const int L = __popcll(kmask);
  const int pos = vs::lanes_below(kmask);
  int32_t* orow_i = dist_ids + static_cast<int64_t>(row) * ld_dist;
  float* orow_p = dist_probs + static_cast<int64_t>(row) * ld_dist;
  if (keep) {
    orow_i[pos] = tok;
    orow_p[pos] = prob;
  }
  if (lane >= L && lane < M) {  // pad the rest of the row
    orow_i[lane] = -1;
    orow_p[lane] = 0.f;
  }
  if (lane == 0) dist_len[row] = L;

  if (u != nullptr) {
    // draw over the kept candidates in pool order, from the stored fp32 probs;
    // kept lanes are in increasing order, so lane order is slot order
    const double w = keep ? static_cast<double>(prob) : 0.0;
    int32_t pick = -1;
    if (L > 0) {
      // kept lanes lie below the last kept lane + 1
      const int nl = 64 - __clzll(static_cast<long long>(kmask));
      // lanes of weight 0 are skipped: they add nothing and are never the
      // first lane to pass
      const bool live = lane < nl && w != 0.0;
      vs::wave_lds_sync();  // the first scan's slots have been read
      double acc = 0.0;
      for (uint64_t m = __ballot(live); m; m &= m - 1) {
        const int j = __ffsll(static_cast<long long>(m)) - 1;
        acc += vs::bcast(w, j);
        if (lane == 0) run[j] = acc;
      }
      vs::wave_lds_sync();
      const double mine = live ? run[lane] : 0.0;
      const double target = static_cast<double>(u[row]) * acc;
      const uint64_t hit = __ballot(keep && target < mine);
      int src;
      if (hit) {
        src = __ffsll(static_cast<long long>(hit)) - 1;
      } else {
        const uint64_t posm = __ballot(keep && w > 0.0);
        src = posm ? 63 - __clzll(static_cast<long long>(posm)) : (__ffsll(static_cast<long long>(kmask)) - 1);
      }
      pick = vs::bcast(tok, src);
    }
    if (lane == 0) drawn[row] = pick;
  }
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
  const int k_eff = top_k < 0 ? 20 : (top_k == 0 ? VS_POOL : (top_k < VS_POOL ? top_k : VS_POOL));
  const int blocks = (rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  policy_kernel<<<dim3(blocks), dim3(64 * ROWS_PER_BLOCK), 0, stream>>>(
      vals, ids, ld, rows, M, temperature, k_eff, top_p, min_p, dist_ids, dist_probs, dist_len,
      ld_dist, u, drawn);
  return vs::check_launch();
}
