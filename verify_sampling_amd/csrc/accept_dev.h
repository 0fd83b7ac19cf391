// Acceptance of one speculative window b, for one 64-lane wave (see
// accept.hip for the rules of every mode).  run: 64 LDS doubles of this
// wave.  The distribution pointers may address global or LDS memory.
#pragma once

#include "wave_ops.h"

namespace {

struct Dists {
  const int32_t* p_ids;
  const float* p_probs;
  const int32_t* p_len;
  int p_ld;
  int64_t p_ws;
  const int32_t* q_ids;
  const float* q_probs;
  const int32_t* q_len;
  int q_ld;
  int64_t q_ws;
};

__device__ __forceinline__ int clamp_len(int n, int ld) { return n < 0 ? 0 : (n > ld ? ld : n); }

// Total probability of token x over the lanes [0, n) of a sparse row: the
// entries holding x, summed in lane order (one entry in a well-formed row).
__device__ __forceinline__ double prob_of(int32_t id, double p, int n, int32_t x) {
  const int lane = threadIdx.x & 63;
  uint64_t m = __ballot(lane < n && id == x);
  double s = 0.0;
  while (m) {
    s += vs::bcast(p, __ffsll(static_cast<long long>(m)) - 1);
    m &= m - 1;
  }
  return s;
}

__device__ __forceinline__ void accept_window(int mode, int b, int k, const Dists& d,
                                              const int32_t* __restrict__ drafts,
                                              const int32_t* __restrict__ parent,
                                              const float* __restrict__ u, int32_t* __restrict__ out_tokens,
                                              int32_t* __restrict__ out_n, double* run) {
  const int lane = threadIdx.x & 63;
  const int32_t* dr = drafts + static_cast<int64_t>(b) * k;
  int32_t my_tok = -1;  // lane j holds emitted token j
  int n = 0;

  if (mode == VS_ACCEPT_GREEDY) {
    bool done = false;
    for (int i = 0; i < k && !done; ++i) {
      const int32_t a = d.p_ids[(static_cast<int64_t>(b) * d.p_ws + i) * d.p_ld];
      const int32_t x = dr[i];
      if (lane == n) my_tok = (x == a) ? x : a;
      ++n;
      done = x != a;
    }
    if (!done) {
      const int32_t a = d.p_ids[(static_cast<int64_t>(b) * d.p_ws + k) * d.p_ld];
      if (lane == n) my_tok = a;
      ++n;
    }
  } else if (mode == VS_ACCEPT_GREEDY_TREE) {
    const int32_t* par = parent + static_cast<int64_t>(b) * k;
    uint64_t agree = 0;
    int my_depth = 0;  // lane j: depth of node j (root children have depth 1)
    for (int j = 0; j < k; ++j) {
      const int32_t pj = par[j];
      const bool valid = pj >= -1 && pj < j;  // a malformed parent never agrees
      const int prow = pj < 0 ? 0 : pj + 1;
      const int32_t a = valid ? d.p_ids[(static_cast<int64_t>(b) * d.p_ws + prow) * d.p_ld] : -1;
      const bool pok = pj == -1 || (valid && ((agree >> pj) & 1ull));
      if (valid && pok && dr[j] == a) agree |= 1ull << j;
      const int dpar = (valid && pj >= 0) ? vs::bcast(my_depth, pj) : 0;
      if (lane == j) my_depth = dpar + 1;
    }
    // deepest agreeing node, lowest number on a tie
    int keyv = ((agree >> lane) & 1ull) && lane < k ? my_depth * 64 + (63 - lane) : -1;
    for (int off = 32; off > 0; off >>= 1) {
      const int o = __shfl_xor(keyv, off, 64);
      keyv = o > keyv ? o : keyv;
    }
    const int best = keyv < 0 ? -1 : 63 - (keyv & 63);
    const int depth = keyv < 0 ? 0 : keyv >> 6;
    int node = best;
    for (int pos = depth - 1; pos >= 0; --pos) {
      if (lane == pos) my_tok = dr[node];
      node = par[node];
    }
    n = depth;
    const int last_row = best < 0 ? 0 : best + 1;
    const int32_t a = d.p_ids[(static_cast<int64_t>(b) * d.p_ws + last_row) * d.p_ld];
    if (lane == n) my_tok = a;
    ++n;
  } else if (mode == VS_ACCEPT_NAIVE) {
    const float* ub = u + static_cast<int64_t>(b) * (k + 1) * 2;
    for (int i = 0; i <= k; ++i) {
      const int64_t prow = static_cast<int64_t>(b) * d.p_ws + i;
      const int pl = clamp_len(d.p_len[prow], d.p_ld);
      const int32_t pid = lane < pl ? d.p_ids[prow * d.p_ld + lane] : -1;
      const double pp = lane < pl ? static_cast<double>(d.p_probs[prow * d.p_ld + lane]) : 0.0;
      const int32_t x = vs::bcast(pid, vs::seq_draw(pp, pl, ub[2 * i + 1], run));  // -1 if p is empty
      if (lane == n) my_tok = x;
      ++n;
      if (i == k || x < 0 || x != dr[i]) break;  // an empty row's -1 always ends the window
    }
  } else if (mode == VS_ACCEPT_NAIVE_TREE) {
    // walk from the root: draw at the current row, move to the child carrying
    // the draw (lowest number if siblings repeat a token); node numbers only
    // grow along the walk, so it emits at most k + 1 tokens
    const int32_t* par = parent + static_cast<int64_t>(b) * k;
    const float* ub = u + static_cast<int64_t>(b) * (k + 1) * 2;
    const int32_t my_par = lane < k ? par[lane] : -2;
    const int32_t my_tk = lane < k ? dr[lane] : -1;
    const bool node_ok = lane < k && my_par >= -1 && my_par < lane;  // malformed nodes are unreachable
    int node = -1, row = 0;
    for (int step = 0; step <= k; ++step) {
      const int64_t prow = static_cast<int64_t>(b) * d.p_ws + row;
      const int pl = clamp_len(d.p_len[prow], d.p_ld);
      const int32_t pid = lane < pl ? d.p_ids[prow * d.p_ld + lane] : -1;
      const double pp = lane < pl ? static_cast<double>(d.p_probs[prow * d.p_ld + lane]) : 0.0;
      const int32_t x = vs::bcast(pid, vs::seq_draw(pp, pl, ub[2 * row + 1], run));
      if (lane == n) my_tok = x;
      ++n;
      if (x < 0) break;
      const uint64_t m = __ballot(node_ok && my_par == node && my_tk == x);
      if (m == 0) break;
      node = __ffsll(static_cast<long long>(m)) - 1;
      row = node + 1;
    }
  } else if (mode == VS_ACCEPT_POINT_MASS) {
    const float* ub = u + static_cast<int64_t>(b) * (k + 1) * 2;
    bool stopped = false;
    for (int i = 0; i < k && !stopped; ++i) {
      const int64_t prow = static_cast<int64_t>(b) * d.p_ws + i;
      const int pl = clamp_len(d.p_len[prow], d.p_ld);
      const int32_t pid = lane < pl ? d.p_ids[prow * d.p_ld + lane] : -1;
      const double pp = lane < pl ? static_cast<double>(d.p_probs[prow * d.p_ld + lane]) : 0.0;
      const int32_t x = dr[i];
      if (static_cast<double>(ub[2 * i]) < prob_of(pid, pp, pl, x)) {  // u * q(x), q(x) = 1
        if (lane == n) my_tok = x;
        ++n;
        continue;
      }
      // (p - delta(x))+ is p without x
      const double r = (lane < pl && pid != x) ? pp : 0.0;
      const double z = vs::seq_sum(r, pl);
      const int j = z > 0.0 ? vs::seq_draw(r, pl, ub[2 * i + 1], run) : vs::seq_draw(pp, pl, ub[2 * i + 1], run);
      const int32_t t = vs::bcast(pid, j);
      if (lane == n) my_tok = t;
      ++n;
      stopped = true;
    }
    if (!stopped) {  // bonus draw from p_k
      const int64_t prow = static_cast<int64_t>(b) * d.p_ws + k;
      const int pl = clamp_len(d.p_len[prow], d.p_ld);
      const int32_t pid = lane < pl ? d.p_ids[prow * d.p_ld + lane] : -1;
      const double pp = lane < pl ? static_cast<double>(d.p_probs[prow * d.p_ld + lane]) : 0.0;
      const int32_t t = vs::bcast(pid, vs::seq_draw(pp, pl, ub[2 * k + 1], run));
      if (lane == n) my_tok = t;
      ++n;
    }
  } else {  // sampled chain
    const float* ub = u + static_cast<int64_t>(b) * (k + 1) * 2;
    bool stopped = false;
    for (int i = 0; i < k && !stopped; ++i) {
      const int64_t prow = static_cast<int64_t>(b) * d.p_ws + i;
      const int64_t qrow = static_cast<int64_t>(b) * d.q_ws + i;
      const int pl = clamp_len(d.p_len[prow], d.p_ld);
      const int ql = clamp_len(d.q_len[qrow], d.q_ld);
      const int32_t pid = lane < pl ? d.p_ids[prow * d.p_ld + lane] : -1;
      const double pp = lane < pl ? static_cast<double>(d.p_probs[prow * d.p_ld + lane]) : 0.0;
      const int32_t qid = lane < ql ? d.q_ids[qrow * d.q_ld + lane] : -1;
      const double qp = lane < ql ? static_cast<double>(d.q_probs[qrow * d.q_ld + lane]) : 0.0;
      const int32_t x = dr[i];
      const double px = prob_of(pid, pp, pl, x);
      const double qx = prob_of(qid, qp, ql, x);
      if (static_cast<double>(ub[2 * i]) * qx < px) {  // accept d_i
        if (lane == n) my_tok = x;
        ++n;
        continue;
      }
      // residual (p - q)+ over p's support, in p's order
      double qt = 0.0;
      for (int j = 0; j < ql; ++j) {
        const int32_t t = vs::bcast(qid, j);
        const double pj = vs::bcast(qp, j);
        if (t == pid) qt += pj;
      }
      const double diff = pp - qt;
      const double r = (lane < pl && diff > 0.0) ? diff : 0.0;
      const double z = vs::seq_sum(r, pl);
      const int j = z > 0.0 ? vs::seq_draw(r, pl, ub[2 * i + 1], run) : vs::seq_draw(pp, pl, ub[2 * i + 1], run);
      const int32_t t = vs::bcast(pid, j);
      if (lane == n) my_tok = t;
      ++n;
      stopped = true;
    }
    if (!stopped) {  // bonus draw from p_k
      const int64_t prow = static_cast<int64_t>(b) * d.p_ws + k;
      const int pl = clamp_len(d.p_len[prow], d.p_ld);
      const int32_t pid = lane < pl ? d.p_ids[prow * d.p_ld + lane] : -1;
      const double pp = lane < pl ? static_cast<double>(d.p_probs[prow * d.p_ld + lane]) : 0.0;
      const int j = vs::seq_draw(pp, pl, ub[2 * k + 1], run);
      const int32_t t = vs::bcast(pid, j);
      if (lane == n) my_tok = t;
      ++n;
    }
  }

  int32_t* out = out_tokens + static_cast<int64_t>(b) * (k + 1);
  if (lane <= k) out[lane] = lane < n ? my_tok : -1;
  if (lane == 0) out_n[b] = n;
}

}  // namespace
