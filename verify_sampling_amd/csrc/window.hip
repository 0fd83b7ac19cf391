// verify_window: the acceptance stage of one verify window in two launches;
// verify_tree_window: the same for a token tree.
//
// "Speculative decoding on RDNA": §04 (every verify row, and the draft's
// candidates for it, penalised against H_i, the last W tokens of prompt ||
// emitted || drafts[0, i); only the penalised row leaves the GPU), §03 "how
// hipfire does it" (the 64-wide pool, then temperature, top-k, min-p and
// top-p; the same policy for the draft's re-scored candidates), §03 steps
// 1-4 and §02 (rejection sampling, greedy acceptance).
//
// The same work as penalize_rows (target rows and candidates), topk_rows
// (K = 64), sample_policy_rows (p and q) and spec_accept_rows (sampled or
// greedy), with the same device code for every stage, so the same bits, in
// two launches instead of seven:
//  * select: one wave per (row, 1024- or 4096-element chunk) of the target
//    rows.  The chunk's values are loaded, the row's penalties are applied to
//    those of its history tokens that fall in the chunk (in the registers,
//    and written back to the row, which is penalised in place), then the
//    chunk's top 64 are selected as topk_rows does.  Extra waves, one per
//    draft row, penalise its candidates against the same history and compute
//    the draft's policy distribution.
//  * finish: one wave per row, in workgroups of eight; each wave merges its
//    row's chunk lists into the pool and runs the target's policy on it,
//    while the draft distributions, uniforms and drafts loaded at the start
//    wait in registers; then one wave accepts the drafts (in the last
//    workgroup to finish, when there are several).  Pools and distributions
//    pass through LDS and are also written out.
// Both stages are latency-bound (one window is a few MB): the select stage's
// cost is its waves' load latency and selection, the finish stage's a
// single wave's dependent merge, policy and acceptance per row.
//
// A token tree ("One RDNA4 verify pass has slack for about two dozen
// speculative tokens", "Spend the budget on a tree, not a longer guess":
// several branches sharing a prefix, each attending only to its ancestors)
// takes the same two launches as penalize_tree_rows, topk_rows,
// sample_policy_rows and spec_accept_rows (naive-sampling or greedy tree
// walk) would: row 0 is the root, row 1 + j node j, and each row's history
// is the context followed by its own branch's path, which each select wave
// builds in its lanes from the nodes' parents (loaded with the chunk).

#include "accept_dev.h"
#include "penalty_dev.h"
#include "policy_dev.h"
#include "topk_dev.h"

namespace {

constexpr int WIN_K = VS_POOL;     // pool width
constexpr int FIN_WAVES = 8;       // waves of the finish workgroup
constexpr int MAX_WIN_ROWS = VS_MAX_DRAFTS + 1;

// H_row for every row: the last `window` tokens of ctx || drafts[0, min(row, k)).
struct History {
  const int32_t* ctx;
  const int32_t* drafts;
  int ctx_len, k, V, window;

  // H_row's length; start: the position of its first token in ctx || drafts
  __device__ __forceinline__ int span(int row, int64_t& start) const {
    const int nd = row < k ? row : k;
    const int64_t total = static_cast<int64_t>(ctx_len) + nd;
    const int hlen = static_cast<int>(total < window ? total : window);
    start = total - hlen;
    return hlen;
  }
  // token j of a history starting at `start` (-1 for ids outside the
  // vocabulary, which never match)
  __device__ __forceinline__ int32_t token(int64_t start, int j) const {
    const int64_t pos = start + j;
    const int32_t t = pos < ctx_len ? ctx[pos] : drafts[pos - ctx_len];
    return (t >= 0 && t < V) ? t : -1;
  }
};

struct Penalty {
  float rep, pres, freq;
};

struct WinArgs {
  float* logits;  // [R][ld] target rows, penalised in place
  int64_t ld;
  int R;
  History h;      // h.k = R - 1 drafts (a tree: its nodes' tokens)
  const int32_t* parent;  // a tree: node j's parent (-1 = the root); null for a chain
  Penalty pen;
  int mode;       // the acceptance mode (VS_ACCEPT_*)
  bool q_rows;    // the draft's candidates are penalised and scored (a sampled chain)
  bool use_u;     // the acceptance draws
  const int32_t* q_ids;  // [k][q_ld], q_m candidates per row
  const float* q_vals;
  int64_t q_ld;
  int q_m;
  float* q_pen;          // nullable: penalised candidate logits [k][q_ld]
  float temperature;
  int k_eff;
  float top_p, min_p;
  const float* u;        // [R][2]
  float* pool_vals;      // [R][64]
  int32_t* pool_ids;
  int32_t* p_ids;        // [R][64]
  float* p_probs;
  int32_t* p_len;        // [R]
  int32_t* q_dist_ids;   // [k][q_ld]
  float* q_dist_probs;
  int32_t* q_dist_len;   // [k]
  int32_t* out_tokens;   // [R]
  int32_t* out_n;
  uint64_t* ws;
  uint32_t* counter;     // finish workgroups that have published their rows (several workgroups)
  int chunks, lg_jp, lg_j2;
};

// The penalties of one row on its history tokens in [base, base + n).
// tok(j0): the history token at position j0 + lane in each lane (-1 past the
// history's hlen tokens); called with uniform j0 in uniform control flow.
// Each distinct token is handled once, at its first history position, with
// its count over the whole history, by the lane that holds it (element j of
// lane l is chunk index 256 (j / 4) + 4 l + j % 4), which also writes it back
// to the row with a device-coherent store.
template <int NPL, class Tok>
__device__ __forceinline__ void penalize_chunk(float (&x)[NPL], float* xrow, int base, int n, int hlen,
                                               const Tok& tok, const Penalty& pen) {
  const int lane = threadIdx.x & 63;
  for (int h0 = 0; h0 < hlen; h0 += 64) {  // uniform
    const int32_t t = tok(h0);
    uint64_t inr = __ballot(t >= base && t < base + n);
    while (inr) {  // uniform
      const int src = __ffsll(static_cast<long long>(inr)) - 1;
      inr &= inr - 1;
      const int32_t tk = vs::bcast(t, src);
      const int pos = h0 + src;
      bool first = true;
      int c = 0;
      for (int g0 = 0; g0 < hlen; g0 += 64) {  // uniform
        const int32_t tt = g0 == h0 ? t : tok(g0);
        const uint64_t eq = __ballot(tt == tk);
        c += __popcll(eq);
        const int before = pos - g0;  // positions of this batch before pos
        if (before > 0 && (before >= 64 ? eq : (eq & ((1ull << before) - 1ull))) != 0ull) first = false;
      }
      if (!first) continue;
      const int li = tk - base;
      const int owner = (li & 255) >> 2;
      const int jreg = ((li >> 8) << 2) | (li & 3);
      if (lane == owner) {
        float nv = 0.f;
#pragma unroll
        for (int q = 0; q < NPL; ++q) {
          if (q == jreg) {  // uniform: no dynamic register index
            x[q] = penalize_one(x[q], c, pen.rep, pen.pres, pen.freq);
            nv = x[q];
          }
        }
        // (chunk_unit waits for these stores before its exact path reloads the chunk)
        __hip_atomic_store(xrow + tk, nv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// The select stage's hook for a chain: target row `row` against H_row.
struct ChunkPenalty {
  History h;
  Penalty pen;
  int row;
  int32_t t0;  // this lane's token of the history's first 64, loaded with the chunk
  template <int NPL>
  __device__ __forceinline__ void operator()(float (&x)[NPL], float* xrow, int base, int n) const {
    if (h.window == 0) return;
    const int lane = threadIdx.x & 63;
    int64_t start;
    const int hlen = h.span(row, start);
    auto tok = [&](int j0) { return j0 == 0 ? t0 : (j0 + lane < hlen ? h.token(start, j0 + lane) : -1); };
    penalize_chunk(x, xrow, base, n, hlen, tok, pen);
  }
};

// The select stage's hook for a tree: row 0 against the context, row 1 + j
// against the context followed by node j's path from the root.  parv, tokv:
// lane i holds node i's parent and token (lanes past the nodes: -2, -1).
// The path is walked up from node row - 1 while the parent index decreases
// (a parent outside [-1, child) ends it, as in penalize_tree_rows), and its
// tokens are placed root first in the lanes.
struct ChunkPenaltyTree {
  History h;
  Penalty pen;
  int row;
  int32_t parv, tokv;
  int32_t ctxv;  // lane i: context token ctx_len - 64 + i (-1 before the context), loaded with the chunk
  template <int NPL>
  __device__ __forceinline__ void operator()(float (&x)[NPL], float* xrow, int base, int n) const {
    if (h.window == 0) return;
    const int lane = threadIdx.x & 63;
    int len = 0;
    if (row > 0) {  // uniform
      int child = row - 1;
      len = 1;
      int q = __builtin_amdgcn_readlane(parv, child);
      while (q > -1 && q < child) {  // indices strictly decrease: at most row steps
        ++len;
        child = q;
        q = __builtin_amdgcn_readlane(parv, q);
      }
    }
    int32_t pathv = -1;  // lane i: the path's token i
    for (int s = len - 1, child = row - 1; s >= 0; --s) {
      const int32_t tk = __builtin_amdgcn_readlane(tokv, child);
      if (lane == s) pathv = tk;
      child = __builtin_amdgcn_readlane(parv, child);
    }
    const int64_t total = static_cast<int64_t>(h.ctx_len) + len;
    const int hlen = static_cast<int>(total < h.window ? total : h.window);
    const int64_t start = total - hlen;
    // every lane takes part in the shuffles: the path's tokens sit in other
    // lanes, and so does the context's tail when the history fits in 64
    // tokens (all of its context tokens are then among the last 64)
    const bool tail = hlen <= 64;  // uniform
    auto tok = [&](int j0) {
      const int64_t pos = start + j0 + lane;
      const int pi = static_cast<int>(pos - h.ctx_len);
      const int32_t pt = __shfl(pathv, pi >= 0 && pi < 64 ? pi : 0, 64);
      const int ci = pi + 64;  // in [0, 64) for the context's last 64 positions
      const int32_t ct = tail ? __shfl(ctxv, ci >= 0 && ci < 64 ? ci : 0, 64) : -1;
      if (j0 + lane >= hlen) return -1;
      const int32_t t = pos < h.ctx_len ? (tail ? ct : h.ctx[pos]) : pt;
      return (t >= 0 && t < h.V) ? t : -1;
    };
    penalize_chunk(x, xrow, base, n, hlen, tok, pen);
  }
};

// Draft row i: its candidates penalised against H_i, then its policy.
__device__ __forceinline__ void draft_row(const WinArgs& a, int i, float* vrow, int32_t* irow, double* run) {
  const int lane = threadIdx.x & 63;
  const bool real = lane < a.q_m;
  const int64_t off = static_cast<int64_t>(i) * a.q_ld + lane;
  const int32_t id = real ? a.q_ids[off] : -1;
  float v = real ? a.q_vals[off] : 0.f;
  if (a.h.window > 0) {
    int64_t start;
    const int hlen = a.h.span(i, start);
    const bool in_vocab = id >= 0 && id < a.h.V;  // other ids (empty slots) are never penalised
    int c = 0;
    for (int h0 = 0; h0 < hlen; h0 += 64) {  // uniform
      const int32_t t = h0 + lane < hlen ? a.h.token(start, h0 + lane) : -1;
      const int nb = hlen - h0 < 64 ? hlen - h0 : 64;
      for (int j = 0; j < nb; ++j) c += vs::bcast(t, j) == id;
    }
    if (real && in_vocab && c > 0) v = penalize_one(v, c, a.pen.rep, a.pen.pres, a.pen.freq);
  }
  if (real) {
    vrow[lane] = v;
    irow[lane] = id;
    if (a.q_pen) a.q_pen[off] = v;
  }
  vs::wave_lds_sync();
  const int64_t drow = static_cast<int64_t>(i) * a.q_ld;
  policy_row(vrow, irow, a.q_m, a.temperature, a.k_eff, a.top_p, a.min_p, a.q_dist_ids + drow,
             a.q_dist_probs + drow, a.q_dist_len + i, nullptr, nullptr, run);
}

struct DraftShared {
  float v[64];
  int32_t id[64];
  double run[64];
};

template <int NPL, bool TREE>
__global__ void __launch_bounds__(64 * WAVES)
window_select_kernel(WinArgs a) {
  __shared__ union {
    WaveShared chunk;
    DraftShared draft;
  } shared[WAVES];
  const int w = vs::wave_index();
  if (a.counter != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *a.counter = 0u;  // read by the next launch
  const int unit = blockIdx.x * WAVES + w;
  const int cunits = a.R * a.chunks;
  if (unit < cunits) {
    const int row = unit / a.chunks, chunk = unit - row * a.chunks;
    const int lane = threadIdx.x & 63;
    if constexpr (TREE) {
      const bool node = lane < a.h.k && a.h.window > 0;
      const int32_t parv = node ? a.parent[lane] : -2;
      const int32_t tokv = node ? a.h.drafts[lane] : -1;
      const int ci = a.h.ctx_len - 64 + lane;
      const int32_t ctxv = a.h.window > 0 && ci >= 0 ? a.h.ctx[ci] : -1;
      chunk_unit<NPL, 4, true>(shared[w].chunk, a.logits, a.ld, row, chunk, a.h.V, WIN_K, a.chunks, a.ws,
                               a.pool_vals, a.pool_ids, WIN_K, ChunkPenaltyTree{a.h, a.pen, row, parv, tokv, ctxv});
    } else {
      int64_t start = 0;
      const int hlen = a.h.window > 0 ? a.h.span(row, start) : 0;
      const int32_t t0 = lane < hlen ? a.h.token(start, lane) : -1;
      chunk_unit<NPL, 4, true>(shared[w].chunk, a.logits, a.ld, row, chunk, a.h.V, WIN_K, a.chunks, a.ws,
                               a.pool_vals, a.pool_ids, WIN_K, ChunkPenalty{a.h, a.pen, row, t0});
    }
  } else if (a.q_rows && unit < cunits + a.h.k) {
    DraftShared& d = shared[w].draft;
    draft_row(a, unit - cunits, d.v, d.id, d.run);
  }
}

__global__ void __launch_bounds__(64 * FIN_WAVES)
window_finish_kernel(WinArgs a) {
  __shared__ MergeShared msh[FIN_WAVES];
  __shared__ float pv[FIN_WAVES][WIN_K];  // each wave's current pool
  __shared__ int32_t pi[FIN_WAVES][WIN_K];
  __shared__ int32_t dids[MAX_WIN_ROWS][WIN_K];
  __shared__ float dprobs[MAX_WIN_ROWS][WIN_K];
  __shared__ int32_t dlen[MAX_WIN_ROWS];
  __shared__ int32_t qids[MAX_WIN_ROWS - 1][WIN_K];
  __shared__ float qprobs[MAX_WIN_ROWS - 1][WIN_K];
  __shared__ int32_t qlen[MAX_WIN_ROWS - 1];
  __shared__ float us[MAX_WIN_ROWS * 2];
  __shared__ int32_t dr[MAX_WIN_ROWS - 1];
  __shared__ int32_t prt[MAX_WIN_ROWS - 1];  // a tree's parents
  __shared__ double run[FIN_WAVES][64];
  const int lane = threadIdx.x & 63;
  const int w = vs::wave_index();
  const int k = a.h.k;

  // the acceptance's other inputs (draft distributions, uniforms, drafts),
  // loaded now and parked in LDS after the merges, so that their latency
  // overlaps the merges instead of following them (draft rows past the
  // first QPRE of each wave, windows of more than 16 drafts, are loaded
  // when they are parked)
  constexpr int QSLOTS = (MAX_WIN_ROWS - 1 + FIN_WAVES - 1) / FIN_WAVES;
  constexpr int QPRE = 2;
  int32_t qi_r[QPRE], ql_r[QPRE];
  float qp_r[QPRE];
  const bool qm = a.q_rows && lane < a.q_m;
#pragma unroll
  for (int t = 0; t < QPRE; ++t) {
    const int i = w + FIN_WAVES * t;
    const bool live = a.q_rows && i < k;
    const int64_t off = static_cast<int64_t>(i) * a.q_ld + lane;
    qi_r[t] = live && qm ? a.q_dist_ids[off] : -1;
    qp_r[t] = live && qm ? a.q_dist_probs[off] : 0.f;
    ql_r[t] = live && lane == 0 ? a.q_dist_len[i] : 0;
  }
  const int tid = static_cast<int>(threadIdx.x);
  const float u_r = a.use_u && tid < 2 * a.R ? a.u[tid] : 0.f;
  const int32_t d_r = tid < k ? a.h.drafts[tid] : 0;
  const int32_t p_r = a.parent != nullptr && tid < k ? a.parent[tid] : -1;

  __shared__ int last;
  // one row per wave: the grid holds ceil(R / FIN_WAVES) workgroups
  const int row = blockIdx.x * FIN_WAVES + w;
  if (row < a.R) {  // uniform per wave
    if (a.chunks > 1) {
      merge_row(msh[w], a.logits, a.ld, row, a.h.V, WIN_K, a.chunks, a.lg_jp, a.lg_j2, a.ws, pv[w], pi[w]);
      vs::wave_lds_sync();
      a.pool_vals[row * WIN_K + lane] = pv[w][lane];
      a.pool_ids[row * WIN_K + lane] = pi[w][lane];
    } else {  // the select stage wrote the pool
      vs::wave_lds_sync();  // the previous row's pool has been read
      pv[w][lane] = a.pool_vals[row * WIN_K + lane];
      pi[w][lane] = a.pool_ids[row * WIN_K + lane];
      vs::wave_lds_sync();
    }
    policy_row(pv[w], pi[w], WIN_K, a.temperature, a.k_eff, a.top_p, a.min_p, dids[row], dprobs[row],
               &dlen[row], nullptr, nullptr, run[w]);
    vs::wave_lds_sync();
    a.p_ids[row * WIN_K + lane] = dids[row][lane];
    a.p_probs[row * WIN_K + lane] = dprobs[row][lane];
    if (lane == 0) a.p_len[row] = dlen[row];
  }
  for (int t = 0; t < QSLOTS; ++t) {
    const int i = w + FIN_WAVES * t;
    if (!(a.q_rows && i < k)) break;  // uniform
    const int64_t off = static_cast<int64_t>(i) * a.q_ld + lane;
    qids[i][lane] = t < QPRE ? qi_r[t < QPRE ? t : 0] : (qm ? a.q_dist_ids[off] : -1);
    qprobs[i][lane] = t < QPRE ? qp_r[t < QPRE ? t : 0] : (qm ? a.q_dist_probs[off] : 0.f);
    if (lane == 0) qlen[i] = t < QPRE ? ql_r[t < QPRE ? t : 0] : a.q_dist_len[i];
  }
  if (tid < 2 * a.R) us[tid] = u_r;
  if (tid < k) {
    dr[tid] = d_r;
    prt[tid] = p_r;
  }
  if (gridDim.x > 1) {  // uniform
    // More than one workgroup: each publishes its rows to the device and is
    // counted; the last to arrive reads the others' rows and accepts.  Each
    // wave's stores have reached the L2 before the barrier; one agent-scope
    // release then writes the L2 back, and the last workgroup's acquire
    // drops stale lines before it reads.  Nothing waits on another
    // workgroup.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t arrived = __hip_atomic_fetch_add(a.counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      last = arrived == gridDim.x - 1u;
    }
    __syncthreads();
    if (!last) return;  // uniform over the workgroup
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    for (int r = w; r < a.R; r += FIN_WAVES) {  // the other workgroups' rows
      if (r / FIN_WAVES == static_cast<int>(blockIdx.x)) continue;  // uniform per wave
      dids[r][lane] = a.p_ids[r * WIN_K + lane];
      dprobs[r][lane] = a.p_probs[r * WIN_K + lane];
      if (lane == 0) dlen[r] = a.p_len[r];
    }
  }
  __syncthreads();
  if (w == 0) {
    const Dists d{&dids[0][0], &dprobs[0][0], dlen, WIN_K, k + 1, &qids[0][0], &qprobs[0][0], qlen, WIN_K, k};
    accept_window(a.mode, 0, k, d, dr, a.parent != nullptr ? prt : nullptr, us, a.out_tokens, a.out_n,
                  run[0]);
  }
}

// The workspace: the chunk lists of rows of several chunks (topk_rows' at
// K = 64), then, for more rows than one finish workgroup takes, a 16-byte
// slot for the arrival counter.
size_t lists_bytes(int R, int V) {
  const Plan p = plan_for(R, V);
  return p.chunks <= 1 ? 0 : static_cast<size_t>(R) * p.chunks * WIN_K * sizeof(uint64_t);
}

template <bool TREE>
int launch_window(const WinArgs& a, const Plan& p, int units, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((units + WAVES - 1) / WAVES)), block(64 * WAVES);
  if (p.small)
    window_select_kernel<16, TREE><<<grid, block, 0, stream>>>(a);
  else
    window_select_kernel<64, TREE><<<grid, block, 0, stream>>>(a);
  int st = vs::check_launch();
  if (st != VS_OK) return st;
  window_finish_kernel<<<dim3(static_cast<unsigned>((a.R + FIN_WAVES - 1) / FIN_WAVES)), dim3(64 * FIN_WAVES), 0,
                         stream>>>(a);
  return vs::check_launch();
}

}  // namespace

extern "C" size_t verify_window_workspace_bytes(int R, int V) {
  if (R < 1 || V < WIN_K) return 0;
  return lists_bytes(R, V) + (R > FIN_WAVES ? 16 : 0);
}

extern "C" int verify_window(float* logits, int64_t ld, int R, int V, const int32_t* ctx, int ctx_len,
                             const int32_t* drafts, int window, float repeat, float presence,
                             float frequency, const int32_t* q_ids, const float* q_vals, int64_t q_ld,
                             int q_m, float* q_pen, float temperature, int top_k, float top_p,
                             float min_p, const float* u, float* pool_vals, int32_t* pool_ids,
                             int32_t* p_ids, float* p_probs, int32_t* p_len, int32_t* q_dist_ids,
                             float* q_dist_probs, int32_t* q_dist_len, int32_t* out_tokens,
                             int32_t* out_n, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  if (!logits || !pool_vals || !pool_ids || !p_ids || !p_probs || !p_len || !out_tokens || !out_n)
    return VS_ERR_NULL;
  if (R < 1 || R > MAX_WIN_ROWS || V < WIN_K || V > VS_MAX_VOCAB || ld < V) return VS_ERR_SHAPE;
  const int k = R - 1;
  if (ctx_len < 0) return VS_ERR_SHAPE;
  if ((ctx_len > 0 && !ctx) || (k > 0 && !drafts)) return VS_ERR_NULL;
  if (window < 0 || window > VS_MAX_WINDOW) return VS_ERR_PARAM;
  if (!(repeat > 0.f) || !__builtin_isfinite(repeat) || !__builtin_isfinite(presence) ||
      !__builtin_isfinite(frequency))
    return VS_ERR_PARAM;
  if (__builtin_isnan(temperature) || __builtin_isinf(temperature) || __builtin_isnan(top_p) ||
      __builtin_isnan(min_p))
    return VS_ERR_PARAM;
  const bool sampled = temperature > 0.f;
  if (sampled) {
    if (!u) return VS_ERR_NULL;
    if (k > 0) {
      if (!q_ids || !q_vals || !q_dist_ids || !q_dist_probs || !q_dist_len) return VS_ERR_NULL;
      if (q_m < 1 || q_m > VS_POOL || q_ld < q_m || q_ld > (1 << 24)) return VS_ERR_SHAPE;
    }
  }
  const size_t need = verify_window_workspace_bytes(R, V);
  if (need > 0 && (!workspace || workspace_bytes < need)) return VS_ERR_WORKSPACE;
  if (need > 0 && !vs::aligned16(workspace)) return VS_ERR_ALIGN;

  const Plan p = plan_for(R, V);
  WinArgs a;
  a.logits = logits;
  a.ld = ld;
  a.R = R;
  // nothing to penalise without a window or a history (as penalize_rows)
  a.h = History{ctx, drafts, ctx_len, k, V, (ctx_len == 0 && k == 0) ? 0 : window};
  a.parent = nullptr;
  a.pen = Penalty{repeat, presence, frequency};
  a.mode = sampled ? VS_ACCEPT_SAMPLED : VS_ACCEPT_GREEDY;
  a.q_rows = sampled;
  a.use_u = sampled;
  a.q_ids = q_ids;
  a.q_vals = q_vals;
  a.q_ld = q_ld;
  a.q_m = q_m;
  a.q_pen = q_pen;
  a.temperature = temperature;
  a.k_eff = policy_k_eff(top_k);
  a.top_p = top_p;
  a.min_p = min_p;
  a.u = u;
  a.pool_vals = pool_vals;
  a.pool_ids = pool_ids;
  a.p_ids = p_ids;
  a.p_probs = p_probs;
  a.p_len = p_len;
  a.q_dist_ids = q_dist_ids;
  a.q_dist_probs = q_dist_probs;
  a.q_dist_len = q_dist_len;
  a.out_tokens = out_tokens;
  a.out_n = out_n;
  a.ws = static_cast<uint64_t*>(workspace);
  a.counter = R > FIN_WAVES
                  ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + lists_bytes(R, V))
                  : nullptr;
  a.chunks = p.chunks;
  merge_reads(p.chunks, WIN_K, a.lg_jp, a.lg_j2);

  const int units = R * p.chunks + (sampled ? k : 0);
  const dim3 grid(static_cast<unsigned>((units + WAVES - 1) / WAVES)), block(64 * WAVES);
  return launch_window<false>(a, p, units, stream);
}

extern "C" int verify_tree_window(float* logits, int64_t ld, int R, int V, const int32_t* ctx, int ctx_len,
                                  const int32_t* tokens, const int32_t* parent, int window, float repeat,
                                  float presence, float frequency, float temperature, int top_k, float top_p,
                                  float min_p, const float* u, float* pool_vals, int32_t* pool_ids,
                                  int32_t* p_ids, float* p_probs, int32_t* p_len, int32_t* out_tokens,
                                  int32_t* out_n, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!logits || !pool_vals || !pool_ids || !p_ids || !p_probs || !p_len || !out_tokens || !out_n)
    return VS_ERR_NULL;
  if (R < 1 || R > MAX_WIN_ROWS || V < WIN_K || V > VS_MAX_VOCAB || ld < V) return VS_ERR_SHAPE;
  const int n = R - 1;  // tree nodes
  if (ctx_len < 0) return VS_ERR_SHAPE;
  if ((ctx_len > 0 && !ctx) || (n > 0 && (!tokens || !parent))) return VS_ERR_NULL;
  if (window < 0 || window > VS_MAX_WINDOW) return VS_ERR_PARAM;
  if (!(repeat > 0.f) || !__builtin_isfinite(repeat) || !__builtin_isfinite(presence) ||
      !__builtin_isfinite(frequency))
    return VS_ERR_PARAM;
  if (__builtin_isnan(temperature) || __builtin_isinf(temperature) || __builtin_isnan(top_p) ||
      __builtin_isnan(min_p))
    return VS_ERR_PARAM;
  const bool sampled = temperature > 0.f;
  if (sampled && !u) return VS_ERR_NULL;
  const size_t need = verify_window_workspace_bytes(R, V);
  if (need > 0 && (!workspace || workspace_bytes < need)) return VS_ERR_WORKSPACE;
  if (need > 0 && !vs::aligned16(workspace)) return VS_ERR_ALIGN;

  const Plan p = plan_for(R, V);
  WinArgs a{};
  a.logits = logits;
  a.ld = ld;
  a.R = R;
  // nothing to penalise without a window or a history (as penalize_tree_rows)
  a.h = History{ctx, tokens, ctx_len, n, V, (ctx_len == 0 && n == 0) ? 0 : window};
  a.parent = parent != nullptr && n > 0 ? parent : nullptr;
  a.pen = Penalty{repeat, presence, frequency};
  a.mode = sampled ? VS_ACCEPT_NAIVE_TREE : VS_ACCEPT_GREEDY_TREE;
  a.q_rows = false;
  a.use_u = sampled;
  a.q_ld = 1;
  a.temperature = temperature;
  a.k_eff = policy_k_eff(top_k);
  a.top_p = top_p;
  a.min_p = min_p;
  a.u = u;
  a.pool_vals = pool_vals;
  a.pool_ids = pool_ids;
  a.p_ids = p_ids;
  a.p_probs = p_probs;
  a.p_len = p_len;
  a.out_tokens = out_tokens;
  a.out_n = out_n;
  a.ws = static_cast<uint64_t*>(workspace);
  a.counter = R > FIN_WAVES
                  ? reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + lists_bytes(R, V))
                  : nullptr;
  a.chunks = p.chunks;
  merge_reads(p.chunks, WIN_K, a.lg_jp, a.lg_j2);
  return launch_window<true>(a, p, R * p.chunks, stream);
}
