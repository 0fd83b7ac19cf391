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

#include "accept_dev.h"

namespace {

constexpr int WINDOWS_PER_BLOCK = 4;

__global__ void __launch_bounds__(64 * WINDOWS_PER_BLOCK)
accept_kernel(int mode, int B, int k, Dists d, const int32_t* __restrict__ drafts,
              const int32_t* __restrict__ parent, const float* __restrict__ u,
              int32_t* __restrict__ out_tokens, int32_t* __restrict__ out_n) {
  __shared__ double scan[WINDOWS_PER_BLOCK][64];  // each wave's running sums for seq_draw
  const int wave = vs::wave_index();
  const int b = blockIdx.x * WINDOWS_PER_BLOCK + wave;
  if (b >= B) return;  // whole wave; no block-wide barriers
  accept_window(mode, b, k, d, drafts, parent, u, out_tokens, out_n, scan[wave]);
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
