// verify_windows: the sampled acceptance stage of a batch of windows, each
// window with its own k + 1 target rows and k draft rows over a vocabulary
// of at most 4096 tokens, in one or two launches.
//
// "Speculative decoding on RDNA", §03 "how hipfire does it" (the 64-wide
// pool, then temperature, top-k, min-p and top-p; the same policy for the
// draft) and §03 steps 1-4 (the drafts are draws from q; each is accepted
// with min(1, p/q), else the window ends with a draw from the renormalised
// residual (p - q)+; after k acceptances a bonus draw from p).
//
// The same work as topk_rows (K = 64) and sample_policy_rows on the target
// rows, the same two on the draft rows with one uniform each (the draws are
// the drafts), then spec_accept_rows (VS_ACCEPT_SAMPLED), with the same
// device code for every stage, so the same bits.  A row of at most 4096
// values is a single top-K chunk, so the chunk's sorted list is the row's
// pool, and it goes from the selection to the policy through LDS.
//  * Windows of at most eight rows (k <= 3) in batches of up to 1024: one
//    launch, one workgroup per window and one wave per row.  Each wave
//    selects its row's pool into LDS and runs the policy into the window's
//    distributions in LDS (a draft row's wave also draws the draft); the
//    last wave to finish (an arrival count in LDS) accepts, the others end
//    as soon as their row is done.
//  * Larger batches, and longer windows: two launches.  The rows: one wave
//    per row in workgroups of four independent waves (no barrier), pool in
//    LDS, distribution (and draft) to memory.  The acceptance: one wave per
//    window, as spec_accept_rows.
// Why both (MI355X, k = 3, vocabulary 4096, back-to-back calls): one launch
// took 28-32 us for 1-256 windows against 29-35 us for two, but 0.148 ms
// against 0.116 for 4096 windows and 0.485-0.520 against 0.403-0.406 for
// 16384: a window's waves start and load together and then compute
// together, so a CU's loads and selections overlap less than with
// independent row waves, and the acceptance holds the window's workgroup.
// The five separate calls took 75-78 us for 1-256 windows and 0.132 and
// 0.41-0.42 ms for 4096 and 16384.

#include "accept_dev.h"
#include "policy_dev.h"
#include "topk_dev.h"

namespace {

constexpr int WW_POOL = VS_POOL;       // pool width
constexpr int WW_CHUNK = 64 * 64;      // one top-K chunk of 64 values per lane
constexpr int WW_MAX_DRAFTS = 15;
constexpr int ONE_MAX_ROWS = 8;        // one launch: rows (waves) per window at most
constexpr int ONE_MAX_WINDOWS = 1024;  // one launch: windows at most
constexpr int ROW_WAVES = 4;           // two launches: waves per workgroup

struct WwArgs {
  const float* p;  // [B * (k + 1)][ldp] target logits
  int64_t ldp;
  const float* q;  // [B * k][ldq] draft logits
  int64_t ldq;
  int k, V;
  float temperature;
  int k_eff;
  float top_p, min_p;
  const float* u_draft;  // [B * k]
  const float* u;        // [B][k + 1][2]
  int32_t* drafts;       // [B * k]
  int32_t* p_ids;        // [B * (k + 1)][64]
  float* p_probs;
  int32_t* p_len;        // [B * (k + 1)]
  int32_t* q_ids;        // [B * k][64]
  float* q_probs;
  int32_t* q_len;        // [B * k]
  int32_t* out_tokens;   // [B][k + 1]
  int32_t* out_n;        // [B]
};

// One launch: workgroup = window b, wave r = its row r (target row r for
// r <= k, draft row r - k - 1 after).
__global__ void __launch_bounds__(64 * ONE_MAX_ROWS)
windows_kernel(WwArgs a) {
  __shared__ WaveShared sh[ONE_MAX_ROWS];
  __shared__ float pv[ONE_MAX_ROWS][WW_POOL];
  __shared__ int32_t pi[ONE_MAX_ROWS][WW_POOL];
  __shared__ double run[ONE_MAX_ROWS][64];
  __shared__ int32_t d_ids[ONE_MAX_ROWS][WW_POOL];
  __shared__ float d_probs[ONE_MAX_ROWS][WW_POOL];
  __shared__ int32_t d_len[ONE_MAX_ROWS];
  __shared__ int32_t dr[ONE_MAX_ROWS];
  __shared__ uint32_t arrived;  // waves done with their row
  const int k = a.k;
  const int lane = threadIdx.x & 63;
  const int w = vs::wave_index();  // < 2k + 1 (one wave per row)
  const int64_t b = blockIdx.x;
  if (threadIdx.x == 0) arrived = 0u;
  __syncthreads();

  const bool draft = w > k;
  const int i = draft ? w - k - 1 : w;
  const int64_t grow = draft ? b * k + i : b * (k + 1) + i;
  const float* xrow = draft ? a.q + grow * a.ldq : a.p + grow * a.ldp;
  chunk_unit<64, 4, false>(sh[w], xrow, 0, 0, 0, a.V, WW_POOL, 1, nullptr, pv[w], pi[w], WW_POOL, NoPre{});
  vs::wave_lds_sync();
  policy_row(pv[w], pi[w], WW_POOL, a.temperature, a.k_eff, a.top_p, a.min_p, d_ids[w], d_probs[w], &d_len[w],
             draft ? a.u_draft + grow : nullptr, draft ? &dr[i] : nullptr, run[w]);
  vs::wave_lds_sync();
  int32_t* oi = draft ? a.q_ids : a.p_ids;
  float* op = draft ? a.q_probs : a.p_probs;
  oi[grow * WW_POOL + lane] = d_ids[w][lane];
  op[grow * WW_POOL + lane] = d_probs[w][lane];
  if (lane == 0) {
    (draft ? a.q_len : a.p_len)[grow] = d_len[w];
    if (draft) a.drafts[grow] = dr[i];
  }

  // The last wave to finish its row accepts; the others end here and free
  // their registers for the next windows' waves (a barrier would hold them
  // through the acceptance).  Each wave's LDS writes are complete before its
  // arrival is counted, and the last arriver reads them after its own.
  uint32_t before = 0u;
  if (lane == 0) before = __hip_atomic_fetch_add(&arrived, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
  before = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(before)));
  if (before != static_cast<uint32_t>(2 * k)) return;  // uniform per wave
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const Dists d{&d_ids[0][0], &d_probs[0][0], d_len, WW_POOL, k + 1,
                &d_ids[k + 1][0], &d_probs[k + 1][0], &d_len[k + 1], WW_POOL, k};
  accept_window(VS_ACCEPT_SAMPLED, 0, k, d, dr, nullptr, a.u + b * (k + 1) * 2, a.out_tokens + b * (k + 1),
                a.out_n + b, run[w]);
}

// Two launches, rows: one wave per target or draft row (target rows first),
// four independent waves per workgroup (no barrier).
__global__ void __launch_bounds__(64 * ROW_WAVES)
windows_rows_kernel(WwArgs a, int64_t p_rows, int64_t units) {
  __shared__ WaveShared sh[ROW_WAVES];
  __shared__ float pv[ROW_WAVES][WW_POOL];
  __shared__ int32_t pi[ROW_WAVES][WW_POOL];
  __shared__ double run[ROW_WAVES][64];
  const int w = vs::wave_index();
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * ROW_WAVES + w;
  if (unit >= units) return;  // whole wave; no block-wide barriers
  const bool draft = unit >= p_rows;
  const int64_t row = draft ? unit - p_rows : unit;
  const float* xrow = draft ? a.q + row * a.ldq : a.p + row * a.ldp;
  chunk_unit<64, 4, false>(sh[w], xrow, 0, 0, 0, a.V, WW_POOL, 1, nullptr, pv[w], pi[w], WW_POOL, NoPre{});
  vs::wave_lds_sync();
  if (draft)
    policy_row(pv[w], pi[w], WW_POOL, a.temperature, a.k_eff, a.top_p, a.min_p, a.q_ids + row * WW_POOL,
               a.q_probs + row * WW_POOL, a.q_len + row, a.u_draft + row, a.drafts + row, run[w]);
  else
    policy_row(pv[w], pi[w], WW_POOL, a.temperature, a.k_eff, a.top_p, a.min_p, a.p_ids + row * WW_POOL,
               a.p_probs + row * WW_POOL, a.p_len + row, nullptr, nullptr, run[w]);
}

// Two launches, acceptance: one wave per window.
__global__ void __launch_bounds__(64 * ROW_WAVES)
windows_accept_kernel(WwArgs a, int B) {
  __shared__ double run[ROW_WAVES][64];
  const int w = vs::wave_index();
  const int b = static_cast<int>(blockIdx.x) * ROW_WAVES + w;
  if (b >= B) return;
  const int k = a.k;
  const Dists d{a.p_ids, a.p_probs, a.p_len, WW_POOL, k + 1, a.q_ids, a.q_probs, a.q_len, WW_POOL, k};
  accept_window(VS_ACCEPT_SAMPLED, b, k, d, a.drafts, nullptr, a.u, a.out_tokens, a.out_n, run[w]);
}

}  // namespace

extern "C" int verify_windows(const float* p_logits, int64_t ldp, const float* q_logits, int64_t ldq,
                              int B, int k, int V, float temperature, int top_k, float top_p,
                              float min_p, const float* u_draft, const float* u, int32_t* drafts,
                              int32_t* p_ids, float* p_probs, int32_t* p_len, int32_t* q_ids,
                              float* q_probs, int32_t* q_len, int32_t* out_tokens, int32_t* out_n,
                              hipStream_t stream) {
  if (!p_logits || !u || !out_tokens || !out_n || !p_ids || !p_probs || !p_len) return VS_ERR_NULL;
  if (k > 0 && (!q_logits || !u_draft || !drafts || !q_ids || !q_probs || !q_len)) return VS_ERR_NULL;
  if (B < 1 || B > (1 << 22) || k < 0 || k > WW_MAX_DRAFTS) return VS_ERR_SHAPE;
  if (V < WW_POOL || V > WW_CHUNK || ldp < V || (k > 0 && ldq < V)) return VS_ERR_SHAPE;
  if (__builtin_isnan(temperature) || __builtin_isnan(top_p) || __builtin_isnan(min_p))
    return VS_ERR_PARAM;
  if (__builtin_isinf(temperature)) return VS_ERR_PARAM;
  const WwArgs a{p_logits, ldp, q_logits, ldq, k, V, temperature, policy_k_eff(top_k), top_p, min_p,
                 u_draft, u, drafts, p_ids, p_probs, p_len, q_ids, q_probs, q_len, out_tokens, out_n};
  const int rows = 2 * k + 1;
  if (rows <= ONE_MAX_ROWS && B <= ONE_MAX_WINDOWS) {
    windows_kernel<<<dim3(static_cast<unsigned>(B)), dim3(64 * rows), 0, stream>>>(a);
    return vs::check_launch();
  }
  const int64_t p_rows = static_cast<int64_t>(B) * (k + 1), units = p_rows + static_cast<int64_t>(B) * k;
  windows_rows_kernel<<<dim3(static_cast<unsigned>((units + ROW_WAVES - 1) / ROW_WAVES)), dim3(64 * ROW_WAVES), 0,
                        stream>>>(a, p_rows, units);
  int st = vs::check_launch();
  if (st != VS_OK) return st;
  windows_accept_kernel<<<dim3(static_cast<unsigned>((B + ROW_WAVES - 1) / ROW_WAVES)), dim3(64 * ROW_WAVES), 0,
                          stream>>>(a, B);
  return vs::check_launch();
}
