// The sampler policy of one candidate row, for one 64-lane wave (see
// policy.hip for the definition and the order of every sum).  vrow, irow:
// the row's M <= 64 candidates; orow_i, orow_p: the kept candidates in pool
// order, padded to M with id -1 and probability 0; *len_out: their number.
// u_row (nullable): one uniform, then *drawn_out receives the drawn token.
// run: 64 LDS doubles of this wave.  Every pointer may address global or
// LDS memory.
#pragma once

#include "wave_ops.h"

namespace {

__host__ __device__ inline int policy_k_eff(int top_k) {
  return top_k < 0 ? 20 : (top_k == 0 ? VS_POOL : (top_k < VS_POOL ? top_k : VS_POOL));
}

__device__ __forceinline__ void policy_row(const float* vrow, const int32_t* irow, int M, float temperature,
                                           int k_eff, float top_p, float min_p, int32_t* orow_i,
                                           float* orow_p, int32_t* len_out, const float* u_row,
                                           int32_t* drawn_out, double* run) {
  const int lane = threadIdx.x & 63;
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
  if (keep) {
    orow_i[pos] = tok;
    orow_p[pos] = prob;
  }
  if (lane >= L && lane < M) {  // pad the rest of the row
    orow_i[lane] = -1;
    orow_p[lane] = 0.f;
  }
  if (lane == 0) *len_out = L;

  if (u_row != nullptr) {
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
      const double target = static_cast<double>(*u_row) * acc;
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
    if (lane == 0) *drawn_out = pick;
  }
}

}  // namespace
