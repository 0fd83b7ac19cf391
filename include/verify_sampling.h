/*
 * verify_sampling.h: C ABI of the speculative-decoding verify step on
 * MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [SD]   "Speculative decoding on RDNA" (hipfire 0.4.1 explainer)
 *   [TREE] "One RDNA4 verify pass has slack for about two dozen speculative
 *          tokens"
 *   [PR]   "feat(dflash): developer-only online draft tuning" (hipfire PR #820)
 *
 * Conventions for every entry point:
 *   - Array arguments are DEVICE pointers owned by the caller (the host
 *     functions vs_choose_depth and vs_lookup_tree take host arrays).  The
 *     library allocates no device memory and keeps no mutable global state
 *     apart from a per-thread copy of the last HIP error text (and, for
 *     topk_rows_noalloc, the per-GPU address of its fixed scratch area);
 *     scratch space, where needed, is a caller-provided workspace whose
 *     size a companion *_workspace_bytes() call reports.
 *   - Every call only enqueues work on `stream` and returns; it never
 *     synchronises the device.  Outputs are valid once the stream has
 *     reached the call.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     negative status means nothing was launched and no output was
 *     touched.  VS_ERR_HIP means a launch failed (see
 *     vs_last_error_detail()); in a call of two launches the first may
 *     already be enqueued, and it writes only the workspace.
 *   - Data are never errors: NaN and +-inf logits follow the documented
 *     orders, token ids outside [0, vocab) in a history are ignored.
 *   - Calls on distinct streams with disjoint outputs may run concurrently;
 *     the library is re-entrant.
 */
#ifndef VERIFY_SAMPLING_H
#define VERIFY_SAMPLING_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum vs_status {
  VS_OK = 0,
  VS_ERR_NULL = -1,        /* a required pointer is NULL                     */
  VS_ERR_SHAPE = -2,       /* a size or leading dimension is out of range    */
  VS_ERR_PARAM = -3,       /* a scalar parameter is out of range             */
  VS_ERR_UNSUPPORTED = -4, /* a valid combination the library does not handle */
  VS_ERR_WORKSPACE = -5,   /* workspace missing or too small                 */
  VS_ERR_ALIGN = -6,       /* a pointer or leading dimension is misaligned   */
  VS_ERR_HIP = -7,         /* the HIP runtime reported an error at launch    */
  VS_ERR_SCRATCH = -8      /* the input needs more scratch than the library's
                              fixed per-GPU area holds (topk_rows_noalloc)  */
};

#define VS_ABI_VERSION 6
#define VS_MAX_ROWS 24     /* verify rows R = k + 1 per projection call      */
#define VS_POOL 64         /* width of the sampler's candidate pool          */
#define VS_MAX_WINDOW 4096 /* longest penalty window                         */
#define VS_MAX_VOCAB 262144
#define VS_MAX_DRAFTS 63   /* drafts (or tree nodes) per window: rows = k + 1 <= 64 */

/* ABI version of the loaded library (VS_ABI_VERSION at build time). */
int vs_abi_version(void);

/* Static description of a status code. */
const char* vs_status_string(int status);

/* Text of the last VS_ERR_HIP on the calling thread ("" if none). */
const char* vs_last_error_detail(void);

/*
 * verify_gemv_rows: the multi-row verify projection.
 *   [SD] §01: one verify pass streams each weight matrix once for the
 *   current position plus k drafts (R = k + 1 rows); §02: the multi-row
 *   projections sum in exactly the single-row decode order.
 *
 *   Y[r][n] = sum_k W[n][k] * X[r][k],  0 <= r < R, 0 <= n < N,
 * with bf16 weights, fp32 activations and fp32 accumulation.  Row r of the
 * result is bit-identical to the result of the same call with R = 1 and
 * X = row r: the summation order depends only on N and K.  It also does
 * not depend on the workspace: with or without one the bits are the same.
 * Accuracy: every product is exact and the sum is fp32, within
 * 1e-4 * sum_k |W x| of the exact sum in practice (the tested bound), plus
 * 2^-133 * sum_k |W[n][k]| for subnormal activations, whose bits below
 * 2^-133 (the smallest bf16 subnormal) the exact three-plane split cannot
 * hold.  Non-finite activations follow the sum term by term: an output is
 * NaN if a term is NaN (a NaN activation, or +-inf times a zero weight) or
 * +inf and -inf terms meet, else +-inf if a term is infinite.
 *
 *   W    bf16 bit patterns, row-major [N][ldw] (nn.Linear layout, out x in);
 *        finite values; 16-byte aligned, ldw % 8 == 0, K <= ldw < 2^24.
 *   X    fp32 [R][ldx]; 16-byte aligned, ldx % 4 == 0, K <= ldx < 2^24.
 *   Y    fp32 [R][ldy]; ldy >= N.  Must not overlap W, X or the workspace.
 *   1 <= N <= 2^31 - 1024, 1 <= K with K % 8 == 0, 1 <= R <= VS_MAX_ROWS.
 *   workspace  optional device scratch (16-byte aligned) of at least
 *        verify_gemv_rows_workspace_bytes(N, K, R) bytes.  Some (N, K, R)
 *        run faster with it (partial sums of K partitions are kept there
 *        between two launches); NULL, or a smaller or misaligned buffer,
 *        selects a single-launch path with the same result.  Its contents
 *        on entry do not matter and are overwritten.
 */
size_t verify_gemv_rows_workspace_bytes(int N, int K, int R);
int verify_gemv_rows(const uint16_t* W, int64_t ldw, int N, int K,
                     const float* X, int64_t ldx, int R,
                     float* Y, int64_t ldy,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * penalize_rows: windowed repeat / frequency / presence penalties, in place.
 *   [SD] §04, figure "the penalty history of verify row i":
 *     H_i = last W tokens of (prompt || emitted || drafts[0, i)),
 *   and the draft step proposed for row i is penalised by the same H_i.
 *
 * Row i (0 <= i < rows) uses H_i = the last `window` tokens of
 * (ctx[0, ctx_len) || drafts[0, min(i, n_drafts))).  For each distinct
 * token t in H_i with count c, on its logit l, in fp32 with one rounding
 * per step and in this order:
 *   l = (l > 0) ? l / repeat : l * repeat;   l = l - c * frequency;
 *   l = l - presence.
 * Tokens outside [0, vocab) in H_i are ignored.  window == 0 is a no-op.
 *
 *   Dense  (ids == NULL): logits [rows][ld] holds the whole vocabulary;
 *          width == vocab.
 *   Sparse (ids != NULL): ids [rows][ld] and logits [rows][ld] hold
 *          `width` candidates per row; each candidate slot whose id occurs
 *          in H_i is penalised with that id's count.
 *   ctx     int32 [ctx_len] (may be NULL when ctx_len == 0), the request's
 *           context so far (only its last `window` tokens are read).
 *   drafts  int32 [n_drafts] (may be NULL when n_drafts == 0).
 *   1 <= rows <= 4096, 1 <= width <= ld, 1 <= vocab <= 2^31 - 1,
 *   0 <= window <= VS_MAX_WINDOW, repeat > 0, all parameters finite.
 */
int penalize_rows(float* logits, const int32_t* ids, int64_t ld, int rows, int width,
                  int vocab, const int32_t* ctx, int ctx_len, const int32_t* drafts,
                  int n_drafts, int window, float repeat, float presence, float frequency,
                  hipStream_t stream);

/*
 * penalize_tree_rows: the penalty prepass for the rows of a token tree.
 *   [SD] §04's history rule applied per branch ([TREE] "Spend the budget on
 *   a tree": each branch sees only its own ancestors).  Row 0 is the root
 *   (H = last `window` tokens of ctx); row 1 + j is node j (H = last
 *   `window` tokens of ctx || the tokens on the path from the root down to
 *   node j, inclusive).  The path follows parent[] upwards and stops at -1
 *   or at a parent outside [-1, j).  Otherwise as penalize_rows: the same
 *   penalties, order and rounding, dense (ids == NULL, width == vocab) or
 *   sparse (ids [rows][ld] candidate slots).
 *   logits  fp32 [n_nodes + 1][ld]
 *   tokens, parent  int32 [n_nodes] device arrays (node tokens; parent -1 =
 *           the root), as in spec_accept_rows' tree modes
 *   0 <= n_nodes <= VS_MAX_DRAFTS.
 */
int penalize_tree_rows(float* logits, const int32_t* ids, int64_t ld, int width, int vocab,
                       const int32_t* ctx, int ctx_len, const int32_t* tokens,
                       const int32_t* parent, int n_nodes, int window, float repeat,
                       float presence, float frequency, hipStream_t stream);

/*
 * topk_rows: per-row top-K in the sampler's pool order.
 *   [SD] §03 "how hipfire does it": a 64-wide pool with a fixed tie order;
 *   [PR] "Code map": batched top-K over draft rows, several workgroups per
 *   row, byte-identical with ties, NaN and -inf included.
 *
 * Order: value descending, then index ascending; every NaN ranks below
 * -inf; -0 and +0 are equal.  out_vals holds the input's bits unchanged.
 *   X        fp32 [rows][ldx], V valid entries per row.
 *   out_vals fp32 [rows][ld_out], out_idx int32 [rows][ld_out]; K entries
 *            per row are written.
 *   1 <= rows <= 2^24, 1 <= K <= VS_POOL, K <= V <= VS_MAX_VOCAB, ld_out >= K.
 *   workspace: device memory of at least topk_rows_workspace_bytes(rows, V, K)
 *   bytes, 16-byte aligned; its contents need no initialisation and are
 *   scratch after the call.
 */
size_t topk_rows_workspace_bytes(int rows, int V, int K);
int topk_rows(const float* X, int64_t ldx, int rows, int V, int K,
              float* out_vals, int32_t* out_idx, int64_t ld_out,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * topk_rows_noalloc: topk_rows without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  It allocates nothing:
 * rows of several chunks keep their per-chunk candidate lists in a fixed
 * scratch area of topk_rows_noalloc_max_scratch_bytes() bytes (4 MiB) that
 * the library holds in device memory, one copy per GPU, until the process
 * ends.  Its device address is looked up once per GPU, on the first call
 * made with that GPU current (the library's only other state).
 *   Same arguments, results and errors as topk_rows, bit for bit, and
 *   VS_ERR_SCRATCH, with nothing launched, when topk_rows_workspace_bytes(
 *   rows, V, K) exceeds the scratch size (for example 24 rows of a
 *   151936-token vocabulary at K = 64 need 1.8 MiB and fit).
 *   Every call on one GPU shares that GPU's scratch area, and each call
 *   writes what it later reads (no part of it needs to start at zero):
 *   calls that may overlap on one GPU (distinct streams without ordering,
 *   or several threads) race and must be serialised by the caller.
 */
size_t topk_rows_noalloc_max_scratch_bytes(void);
int topk_rows_noalloc(const float* X, int64_t ldx, int rows, int V, int K,
                      float* out_vals, int32_t* out_idx, int64_t ld_out, hipStream_t stream);

/*
 * sample_policy_rows: the sampler distribution of each row, optionally
 * with one inverse-CDF draw.
 *   [SD] §03 "how hipfire does it": temperature, then top-k (absent means
 *   20 candidates, 0 means the 64-wide pool), then min-p, then top-p, with
 *   the same pool, tie order and summation; q is the same policy applied
 *   to the draft's re-scored candidates.
 *
 * Each row holds M candidates (vals fp32, ids int32; ids < 0 are ignored).
 * They are ordered by (value desc, id asc, NaN last).  temperature <= 0 is
 * greedy (all mass on the first).  Otherwise, in fp64:
 *   weights e_j = exp((l_j - l_0) / T) over the first k_eff candidates,
 *   k_eff = 20 if top_k < 0, 64 if top_k == 0, else min(top_k, 64);
 *   -inf / NaN logits weigh 0 (if l_0 = +inf, each +inf weighs 1);
 *   weight-0 candidates are dropped; min-p keeps e_j >= min_p * e_0;
 *   top-p keeps candidates while the kept mass before them is
 *   < top_p * (total kept mass), at least one (top_p >= 1 keeps all);
 *   sums run sequentially in pool order; p_j = e_j / sum, rounded to fp32.
 *   dist_ids/dist_probs [rows][ld_dist] receive the L kept candidates in
 *   pool order, entries L..M-1 are set to id -1 and probability 0;
 *   dist_len [rows] receives L (>= 1 when any id is >= 0, else 0).
 *   u (fp32 [rows], in [0,1)) and drawn (int32 [rows]) are optional but
 *   must be given together: drawn[r] = dist_ids[r][j], j the first index
 *   with u * total < C_j, C_j the sequential fp64 sum of the fp32 probs.
 *   1 <= M <= VS_POOL, M <= ld, M <= ld_dist, 1 <= rows.
 */
int sample_policy_rows(const float* vals, const int32_t* ids, int64_t ld, int rows, int M,
                       float temperature, int top_k, float top_p, float min_p,
                       int32_t* dist_ids, float* dist_probs, int32_t* dist_len, int64_t ld_dist,
                       const float* u, int32_t* drawn, hipStream_t stream);

/*
 * spec_accept_rows: accept drafts for B windows.
 *   VS_ACCEPT_GREEDY:      [SD] §02: accept the longest prefix of drafts
 *                          equal to the target argmax (p_ids[row][0]); emit
 *                          the argmax at the first mismatch, else the bonus
 *                          argmax of row k ([SD] §01: >= 1 token).
 *   VS_ACCEPT_SAMPLED:     [SD] §03 steps 1-4: accept d_i iff
 *                          u[i][0] * q_i(d_i) < p_i(d_i) (fp64); on
 *                          rejection emit a draw with u[i][1] from
 *                          (p_i - q_i)+ over p_i's support (from p_i if
 *                          that is all zero) and stop; after k acceptances
 *                          emit a bonus draw from p_k with u[k][1].  A
 *                          point-mass q = delta(c) gives [SD] §06.
 *   VS_ACCEPT_POINT_MASS:  deterministic drafts under [SD] §06's rule, the
 *                          sampled test with q_i = delta(d_i) (no q rows):
 *                          accept d_i iff u[i][0] < p_i(d_i); otherwise emit
 *                          a draw with u[i][1] from p_i without d_i,
 *                          renormalised (from p_i if nothing else is left),
 *                          and stop; bonus as in VS_ACCEPT_SAMPLED.  Same
 *                          tokens as VS_ACCEPT_SAMPLED with one-entry q rows.
 *   VS_ACCEPT_NAIVE:       [PR] "Code map", the naive-sampling verify (exact
 *                          for any deterministic draft): row i emits its own
 *                          draw from p_i with u[i][1] and the window goes on
 *                          while that draw equals d_i; after k matches the
 *                          bonus is the draw from p_k with u[k][1].
 *   VS_ACCEPT_NAIVE_TREE:  the naive-sampling verify of a token tree of
 *                          deterministic drafts ([TREE] "Spend the budget on
 *                          a tree"; [PR] "Code map"): starting at the root
 *                          row, emit the row's draw from p with u[row][1];
 *                          if a node whose parent is the current node carries
 *                          that token (the lowest-numbered one), continue at
 *                          its row, else stop.  Rows and nodes as in
 *                          VS_ACCEPT_GREEDY_TREE; a -1 draw (empty row) ends
 *                          the window.
 *   VS_ACCEPT_GREEDY_TREE: [TREE] "Spend the budget on a tree": node j has
 *                          token drafts[j] and parent parent[j] (-1 = root,
 *                          else < j); row 0 is the root, row 1 + j is node
 *                          j.  A node agrees when its token equals its
 *                          parent row's argmax and its parent agrees; the
 *                          deepest agreeing node (lowest number on a tie)
 *                          ends the accepted branch, whose tokens are
 *                          emitted followed by that node's row argmax.
 *
 *   Distributions are sparse rows (ids int32, probs fp32, len int32) as
 *   written by sample_policy_rows.  Window b's row i is row
 *   b * p_win_stride + i of p (p_ld entries per row, p_len[row] valid);
 *   q likewise with q_win_stride (a stride of 0 shares one set of rows
 *   among all windows).  p has k + 1 rows per window, q has k.
 *   drafts  int32 [B][k]   (tree: node tokens)
 *   parent  int32 [B][k]   (tree modes only, else may be NULL)
 *   u       fp32 [B][k+1][2] in [0, 1) (sampled, point-mass and naive modes)
 *           In VS_ACCEPT_NAIVE a draw of -1 (empty row) also ends the window.
 *   q_* may be NULL except in VS_ACCEPT_SAMPLED; p_probs, p_len may be NULL
 *   in the greedy modes.
 *   out_tokens int32 [B][k+1] (entries past the count are -1),
 *   out_n      int32 [B], 1 <= out_n[b] <= k + 1.
 *   1 <= B, 0 <= k <= VS_MAX_DRAFTS, 1 <= p_ld, q_ld <= VS_POOL.
 */
enum vs_accept_mode {
  VS_ACCEPT_SAMPLED = 0,
  VS_ACCEPT_GREEDY = 1,
  VS_ACCEPT_GREEDY_TREE = 2,
  VS_ACCEPT_POINT_MASS = 3,
  VS_ACCEPT_NAIVE = 4,
  VS_ACCEPT_NAIVE_TREE = 5
};
int spec_accept_rows(int mode, int B, int k,
                     const int32_t* p_ids, const float* p_probs, const int32_t* p_len,
                     int p_ld, int64_t p_win_stride,
                     const int32_t* q_ids, const float* q_probs, const int32_t* q_len,
                     int q_ld, int64_t q_win_stride,
                     const int32_t* drafts, const int32_t* parent, const float* u,
                     int32_t* out_tokens, int32_t* out_n, hipStream_t stream);

/*
 * verify_windows: the sampled acceptance stage of B windows in one call,
 * each window with its own k + 1 target rows and k full draft rows over a
 * vocabulary of at most 4096 tokens (the batched sampling workload).
 *   [SD] §03 "how hipfire does it": the 64-wide pool, then temperature,
 *   top-k, min-p and top-p, the same policy for p and q; §03 steps 1-4: the
 *   drafts are draws from q, each accepted with min(1, p/q), else the window
 *   ends with a draw from the renormalised residual (p - q)+, and after k
 *   acceptances comes a bonus draw from p.
 *
 * The same results, bit for bit, as the sequence
 *   topk_rows(p_logits, ldp, B (k + 1), V, 64, pv, pi, 64, ...)
 *   sample_policy_rows(pv, pi, 64, B (k + 1), 64, policy..., p_ids, p_probs,
 *                      p_len, 64, NULL, NULL)
 *   topk_rows(q_logits, ldq, B k, V, 64, qv, qi, 64, ...)
 *   sample_policy_rows(qv, qi, 64, B k, 64, policy..., q_ids, q_probs,
 *                      q_len, 64, u_draft, drafts)
 *   spec_accept_rows(VS_ACCEPT_SAMPLED, B, k, p_ids, p_probs, p_len, 64,
 *                    k + 1, q_ids, q_probs, q_len, 64, k, drafts, NULL, u,
 *                    out_tokens, out_n)
 * with the pools kept on chip: one launch for up to 1024 windows of k <= 3,
 * else two (every row's distribution, then the acceptance).
 *   p_logits fp32 [B (k + 1)][ldp]: window b's target row i is row
 *            b (k + 1) + i; q_logits fp32 [B k][ldq], draft row i of window
 *            b is row b k + i (may be NULL when k = 0).
 *   u_draft  fp32 [B k] in [0, 1): the draw of each draft from its q row
 *            (may be NULL when k = 0); u fp32 [B][k + 1][2] in [0, 1) as
 *            for spec_accept_rows.
 *   Outputs: drafts int32 [B k], the drafts drawn; p_ids, p_probs
 *            [B (k + 1)][64], p_len [B (k + 1)], the target distributions;
 *            q_ids, q_probs [B k][64], q_len [B k], the draft ones (the q
 *            outputs and drafts may be NULL when k = 0); out_tokens int32
 *            [B][k + 1] (entries past the count are -1), out_n int32 [B],
 *            1 <= out_n[b] <= k + 1.
 *   1 <= B <= 2^22, 0 <= k <= 15, 64 <= V <= 4096, ldp >= V, ldq >= V
 *   (k > 0); policy parameters as for sample_policy_rows.  Needs no
 *   workspace.  A VS_ERR_HIP from the second launch leaves the first one's
 *   outputs (distributions and drafts) in place.
 */
int verify_windows(const float* p_logits, int64_t ldp, const float* q_logits, int64_t ldq,
                   int B, int k, int V, float temperature, int top_k, float top_p, float min_p,
                   const float* u_draft, const float* u, int32_t* drafts,
                   int32_t* p_ids, float* p_probs, int32_t* p_len,
                   int32_t* q_ids, float* q_probs, int32_t* q_len,
                   int32_t* out_tokens, int32_t* out_n, hipStream_t stream);

/*
 * verify_window: the whole acceptance stage of one chain window in two
 * launches.
 *   [SD] §04: every verify row, and the draft's candidates for it, are
 *   penalised against H_i before sampling and only the penalised row is
 *   used; §03 "how hipfire does it": the 64-wide pool and the policy, the
 *   same for p and q; §03 steps 1-4 and §02: rejection sampling or greedy
 *   acceptance.
 *
 * The same results, bit for bit, as the sequence
 *   penalize_rows(logits, NULL, ld, R, V, V, ctx, ctx_len, drafts, R - 1, ...)
 *   topk_rows(logits, ld, R, V, 64, pool_vals, pool_ids, 64, ...)
 *   sample_policy_rows(pool_vals, pool_ids, 64, R, 64, policy..., p_ids,
 *                      p_probs, p_len, 64, NULL, NULL)
 *   and, when temperature > 0 (sampled):
 *     penalize_rows(q_vals', q_ids, q_ld, R - 1, q_m, V, ctx, ctx_len,
 *                   drafts, R - 1, ...) on a copy q_vals' written to q_pen
 *     sample_policy_rows(q_vals', q_ids, q_ld, R - 1, q_m, policy...,
 *                        q_dist_ids, q_dist_probs, q_dist_len, q_ld, NULL, NULL)
 *     spec_accept_rows(VS_ACCEPT_SAMPLED, 1, R - 1, p..., 64, R, q..., q_ld,
 *                      R - 1, drafts, NULL, u, out_tokens, out_n)
 *   else (greedy; the draft's candidates, q_* and u are not used and may be NULL):
 *     spec_accept_rows(VS_ACCEPT_GREEDY, 1, R - 1, p..., ...)
 *   logits   fp32 [R][ld], penalised in place (row i against H_i, the last
 *            `window` tokens of ctx || drafts[0, min(i, R - 1)))
 *   ctx      int32 [ctx_len], drafts int32 [R - 1] (device)
 *   q_ids, q_vals  [R - 1][q_ld], q_m candidates per draft row; the inputs
 *            are not changed; q_pen (nullable) receives the penalised values
 *   u        fp32 [R][2] in [0, 1)
 *   pool_vals, pool_ids [R][64]; p_ids, p_probs [R][64], p_len [R];
 *   q_dist_ids, q_dist_probs [R - 1][q_ld], q_dist_len [R - 1];
 *   out_tokens [R] (entries past the count are -1), out_n [1].
 *   1 <= R <= VS_MAX_DRAFTS + 1, 64 <= V <= VS_MAX_VOCAB, ld >= V,
 *   sampled: 1 <= q_m <= VS_POOL, q_m <= q_ld <= 2^24; penalty and policy
 *   parameters as for penalize_rows and sample_policy_rows.
 *   workspace: device memory of at least verify_window_workspace_bytes(R, V)
 *   bytes (the chunk lists of topk_rows at K = 64, and for R > 8 a 16-byte
 *   arrival counter of the finishing workgroups), 16-byte aligned; no
 *   initialisation needed (the call sets what it reads), scratch after the
 *   call.
 *   A VS_ERR_HIP from the second launch leaves the first one's writes in
 *   place: the penalised logits, q_pen, the q distributions and, for
 *   V <= 1024, the pools.
 */
size_t verify_window_workspace_bytes(int R, int V);
int verify_window(float* logits, int64_t ld, int R, int V, const int32_t* ctx, int ctx_len,
                  const int32_t* drafts, int window, float repeat, float presence, float frequency,
                  const int32_t* q_ids, const float* q_vals, int64_t q_ld, int q_m, float* q_pen,
                  float temperature, int top_k, float top_p, float min_p, const float* u,
                  float* pool_vals, int32_t* pool_ids, int32_t* p_ids, float* p_probs,
                  int32_t* p_len, int32_t* q_dist_ids, float* q_dist_probs, int32_t* q_dist_len,
                  int32_t* out_tokens, int32_t* out_n, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * verify_tree_window: the acceptance stage of one token tree in two launches.
 *   [TREE] "Spend the budget on a tree, not a longer guess": one verify pass
 *   checks several branches sharing a prefix, each seeing only its
 *   ancestors; [SD] §04 (each row penalised against its own history before
 *   sampling), §03 (the pool and the policy); [PR] "Code map" (the
 *   naive-sampling verify, walked down the tree).
 *
 * The same results, bit for bit, as the sequence
 *   penalize_tree_rows(logits, NULL, ld, V, V, ctx, ctx_len, tokens, parent,
 *                      R - 1, window, ...)
 *   topk_rows(logits, ld, R, V, 64, pool_vals, pool_ids, 64, ...)
 *   sample_policy_rows(pool_vals, pool_ids, 64, R, 64, policy..., p_ids,
 *                      p_probs, p_len, 64, NULL, NULL)
 *   spec_accept_rows(temperature > 0 ? VS_ACCEPT_NAIVE_TREE : VS_ACCEPT_GREEDY_TREE,
 *                    1, R - 1, p_ids, p_probs, p_len, 64, R, NULL, NULL, NULL,
 *                    1, 0, tokens, parent, u, out_tokens, out_n)
 *   logits   fp32 [R][ld], penalised in place: row 0 (the root) against the
 *            last `window` tokens of ctx, row 1 + j (node j) against the
 *            last `window` of ctx followed by the tokens on the path from
 *            the root down to node j (a parent outside [-1, child) ends the
 *            path, as in penalize_tree_rows)
 *   ctx      int32 [ctx_len]; tokens, parent int32 [R - 1] (device; parent
 *            -1 = the root)
 *   u        fp32 [R][2] in [0, 1) (sampled; may be NULL when greedy)
 *   pool_vals, pool_ids [R][64]; p_ids, p_probs [R][64], p_len [R];
 *   out_tokens [R] (entries past the count are -1), out_n [1].
 *   1 <= R <= VS_MAX_DRAFTS + 1, 64 <= V <= VS_MAX_VOCAB, ld >= V; penalty
 *   and policy parameters as for penalize_tree_rows and sample_policy_rows.
 *   workspace: as for verify_window, verify_window_workspace_bytes(R, V)
 *   bytes, 16-byte aligned, no initialisation needed, scratch after the call.
 *   A VS_ERR_HIP from the second launch leaves the first one's writes in
 *   place: the penalised logits and, for V <= 1024, the pools.
 */
int verify_tree_window(float* logits, int64_t ld, int R, int V, const int32_t* ctx, int ctx_len,
                       const int32_t* tokens, const int32_t* parent, int window, float repeat,
                       float presence, float frequency, float temperature, int top_k, float top_p,
                       float min_p, const float* u, float* pool_vals, int32_t* pool_ids, int32_t* p_ids,
                       float* p_probs, int32_t* p_len, int32_t* out_tokens, int32_t* out_n,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tree_attention_rows: attention of a token tree's verify rows under the tree
 * mask.
 *   [TREE] "Spend the budget on a tree, not a longer guess": one verify pass
 *   carries several branches that share a prefix, with a tree-shaped
 *   attention mask under which each branch attends only to its ancestors;
 *   "Where the tree earns its keep": the candidates' keys and values sit in
 *   scratch slots; "What I am building toward": the mask folded into the
 *   decode attention.
 *
 * Row 0 is the root (the current position; its key and value in scratch
 * slot 0), row 1 + j is node j (slot 1 + j).  Row r attends to the context
 * positions [0, ctx_len) of the cache and to the slots of its ancestors and
 * itself; node j's path follows parent[] up to the root and stops at a
 * parent outside [-1, child).  For query head h (KV head h / (Hq / Hkv)):
 *   out[r][h] = sum_j softmax_j(scale * q[r][h] . k_j) * v_j
 * over those keys, in fp32 arithmetic: exact products (queries and
 * probabilities split into three bf16 pieces), fp32 sums in a fixed order,
 * online softmax over 64-key blocks merged in a fixed order.
 *   q        fp32 [R][Hq][D] contiguous, 16-byte aligned
 *   k_cache, v_cache  bf16 bits [Hkv][cache_len][D] (may be NULL when ctx_len == 0)
 *   k_scr, v_scr      bf16 bits [Hkv][scr_len][D], scr_len >= R
 *   parent   int32 [R - 1] device array (node j's parent; -1 = the root)
 *   out      fp32 [R][Hq][D] contiguous
 *   D == 128, 1 <= R <= 64, Hq % Hkv == 0, (Hq / Hkv) * R <= 256,
 *   0 <= ctx_len <= cache_len, scale finite.
 *   workspace  device memory of at least tree_attention_rows_workspace_bytes(
 *   R, Hq, Hkv, ctx_len) bytes, 16-byte aligned: per-split partial results
 *   (written before they are read; no initialisation needed).
 */
size_t tree_attention_rows_workspace_bytes(int R, int Hq, int Hkv, int ctx_len);
int tree_attention_rows(const float* q, int R, int Hq, int D, const uint16_t* k_cache,
                        const uint16_t* v_cache, int64_t cache_len, int ctx_len,
                        const uint16_t* k_scr, const uint16_t* v_scr, int scr_len,
                        const int32_t* parent, int Hkv, float scale, float* out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * tree_commit_kv: keep the accepted branch.
 *   [TREE] "Where the tree earns its keep": only the accepted branch's keys
 *   and values are kept.
 * For every KV head, scratch slot path[i] is copied to cache position
 * ctx_len + i (0 <= i < n_path), bits unchanged; nothing else changes.
 * path is a device array of slot indices, root first (slot 0, then the
 * slots 1 + j of the accepted nodes in order); an index outside [0,
 * scr_len) leaves its position unchanged.
 *   caches bf16 bits [Hkv][cache_len][D], scratch [Hkv][scr_len][D], all
 *   16-byte aligned; D % 8 == 0; ctx_len + n_path <= cache_len;
 *   0 <= n_path <= 64.
 */
int tree_commit_kv(uint16_t* k_cache, uint16_t* v_cache, int64_t cache_len, int ctx_len,
                   const uint16_t* k_scr, const uint16_t* v_scr, int scr_len,
                   const int32_t* path, int n_path, int Hkv, int D, hipStream_t stream);

/*
 * vs_choose_depth: the draft depth of the next window.
 *   [SD] §05 "What a verify row costs on RDNA": pick the depth k that
 *   maximises the expected emitted tokens (1 plus the running products of
 *   the per-depth acceptance rates) per unit of window cost; k = 0 is one
 *   token per plain decode step, the fallback.
 *
 *   E(k)  = 1 + sum_{j=1..k} prod_{i=1..j} alpha[i-1]   (fp64, increasing j)
 *   rate  = E(k) / cost[k]          (cost[r-1]: cost of a window of r rows)
 * Returns k* in [0, kmax], the depth with the largest rate (the smaller k
 * on a tie), and writes its rate to *rate when rate is not NULL; or a
 * negative status.  Host function: no device work, no stream.
 *   alpha  [kmax] acceptance probability of draft j given drafts 1..j-1
 *          were accepted, each in [0, 1] (may be NULL when kmax == 0)
 *   cost   [kmax + 1] window costs, finite and > 0 (any unit, e.g. the
 *          measured ms of a verify pass of r rows)
 *   0 <= kmax <= VS_MAX_DRAFTS.
 */
int vs_choose_depth(const double* alpha, int kmax, const double* cost, double* rate);

/*
 * vs_lookup_tree: prompt-lookup drafting of a token tree.
 *   [TREE] the introduction (prompt lookup proposes what followed an earlier
 *   occurrence of the last n-gram), "Spend the budget on a tree" and "What I
 *   am building toward" (keep the top few matches, ranked by how often they
 *   recur, as branches sharing a prefix, within one verify pass's budget).
 *
 * Query: the last n tokens of ctx.  Every earlier position p (p + n <
 * ctx_len) with ctx[p, p+n) equal to the query proposes the continuation
 * ctx[p+n, p+n+depth) (shorter where ctx ends).  Identical proposals are one
 * branch whose count is the number of matches proposing it; branches rank by
 * count, then most recent match first.  The top `branches` are merged into a
 * trie: walking each from the root in rank order, an existing child with the
 * same token is shared, otherwise node `nodes++` is appended with its parent
 * (-1 = the root, i.e. the current position).  Node j's parent is < j: the
 * layout spec_accept_rows takes in VS_ACCEPT_GREEDY_TREE mode (tokens as
 * drafts, parent as parent).  Nodes stop at max_nodes.
 *   ctx     int32 [ctx_len] HOST array (token ids); may be NULL if ctx_len == 0
 *   tokens, parent  int32 [max_nodes] HOST arrays, written
 *   1 <= n, 1 <= branches, 1 <= depth, 1 <= max_nodes <= VS_MAX_DRAFTS.
 * Returns the number of nodes (0: no earlier match) or a negative status.
 * Host function: no device work, no stream; uses temporary host memory.
 */
int vs_lookup_tree(const int32_t* ctx, int ctx_len, int n, int branches, int depth,
                   int max_nodes, int32_t* tokens, int32_t* parent);

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_SAMPLING_H */
