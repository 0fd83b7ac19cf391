// spec_accept_rows: acceptance of B speculative windows.
//
// Greedy chain: "Speculative decoding on RDNA", §02 (longest prefix of drafts
// equal to the target argmax) and §01 (the window emits the target's choice
// at the first disagreement, or a bonus token; always >= 1 token).
// Sampled chain: §03 steps 1-4 (accept with min(1, p/q), else a draw from the
// renormalised residual (p - q)+ and stop; bonus draw from p after k
// acceptances); a point-mass q gives §06's takeover rule.
// Deterministic drafts: the point-mass rule of §06 (the sampled test with
// q = delta(d), no q rows needed), and the naive-sampling verify named in the
// "Code map" of "feat(dflash): developer-only online draft tuning" (each row
// emits its own draw from p; the window goes on while the draw equals the
// draft).
// Sampled tree (deterministic drafts such as prompt-lookup trees): the naive
// verify walked down the tree, each row's own draw deciding which child, if
// any, the walk enters.
// Greedy tree: "One RDNA4 verify pass has slack for about two dozen
// speculative tokens", "Spend the budget on a tree": the longest branch the
// target agrees with is accepted.
//
// One 64-lane wave per window.  Rows of a window are processed in order;
// within a row the lanes hold the entries of the sparse distributions.
// Probabilities are fp32 inputs and every decision is taken in fp64: the
// accept test u * q(x) < p(x) is exact (a product of two fp32 values fits in
// fp64), and every sum is sequential in entry order.

#include "wave_ops.h"

namespace {

constexpr int WINDOWS_PER_BLOCK = 4;

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

__global__ void __launch_bounds__(64 * WINDOWS_PER_BLOCK)
accept_kernel(int mode, int B, int k, Dists d, const int32_t* __restrict__ drafts,
              const int32_t* __restrict__ parent, const float* __restrict__ u,
              int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_n) {
  __shared__ double scan[WINDOWS_PER_BLOCK][64];  // each wave's running sums for seq_draw
  const int lane = threadIdx.x & 63;
  const int wave = vs::wave_index();
  const int b = blockIdx.x * WINDOWS_PER_BLOCK + wave;
  if (b >= B) return;  // whole wave; no block-wide barriers
  double* run = scan[wave];

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

extern "C" int spec_accept_rows(int mode, int B, int k, const int32_t* p_ids, const float* p_probs,
                                const int32_t* p_len, int p_ld, int64_t p_win_stride,
                                const int32_t* q_ids, const float* q_probs, const int32_t* q_len,
                                int q_ld, int64_t q_win_stride, const int32_t* drafts,
                                const int32_t* parent, const float* u, int32_t* out_tokens,
                                int32_t* out_n, hipStream_t stream) {
  if (mode != VS_ACCEPT_SAMPLED && mode != VS_ACCEPT_GREEDY && mode != VS_ACCEPT_GREEDY_TREE &&
      mode != VS_ACCEPT_POINT_MASS && mode != VS_ACCEPT_NAIVE && mode != VS_ACCEPT_NAIVE_TREE)
    return VS_ERR_PARAM;
  if (B < 1 || k < 0 || k > VS_MAX_DRAFTS) return VS_ERR_SHAPE;
  if (!p_ids || !out_tokens || !out_n) return VS_ERR_NULL;
  if (k > 0 && !drafts) return VS_ERR_NULL;
  if (p_ld < 1 || p_ld > VS_POOL || p_win_stride < 0) return VS_ERR_SHAPE;
  if (mode == VS_ACCEPT_GREEDY_TREE && k > 0 && !parent) return VS_ERR_NULL;
  if (mode == VS_ACCEPT_POINT_MASS || mode == VS_ACCEPT_NAIVE || mode == VS_ACCEPT_NAIVE_TREE) {
    if (!p_probs || !p_len || !u) return VS_ERR_NULL;
  }
  if (mode == VS_ACCEPT_NAIVE_TREE && k > 0 && !parent) return VS_ERR_NULL;
  if (mode == VS_ACCEPT_SAMPLED) {
    if (!p_probs || !p_len || !u) return VS_ERR_NULL;
    if (k > 0 && (!q_ids || !q_probs || !q_len)) return VS_ERR_NULL;
    if (k > 0 && (q_ld < 1 || q_ld > VS_POOL || q_win_stride < 0)) return VS_ERR_SHAPE;
  }
  Dists d{p_ids, p_probs, p_len, p_ld, p_win_stride, q_ids, q_probs, q_len, q_ld, q_win_stride};
  const int blocks = (B + WINDOWS_PER_BLOCK - 1) / WINDOWS_PER_BLOCK;
  accept_kernel<<<dim3(blocks), dim3(64 * WINDOWS_PER_BLOCK), 0, stream>>>(mode, B, k, d, drafts,
                                                                           parent, u, out_tokens,
                                                                           out_n);
  return vs::check_launch();
}
