// penalize_rows: the per-row penalty prepass, in place.
//
// "Speculative decoding on RDNA", §04 (figure "the penalty history of verify
// row i"): row i is penalised against H_i = last W tokens of (prompt ||
// emitted || drafts[0, i)); the draft step for row i uses the same H_i.
// penalize_tree_rows: the same rule per branch of a token tree ("One RDNA4
// verify pass has slack for about two dozen speculative tokens", "Spend the
// budget on a tree": each branch sees only its ancestors): row 0 is the root
// (history = the context), row 1 + j is node j (history = context || the
// tokens on the path from the root down to node j).
//
// One workgroup per row.  The row's history (<= VS_MAX_WINDOW ids) is staged
// in LDS; each thread owns history positions (dense mode) or candidate slots
// (sparse mode).  In sparse mode the slots are taken up to 256 at a time,
// each by 256 / (slots in the chunk) threads that count its id over
// interleaved shares of the history; the shares' counts are added in LDS.
// In dense mode a
// short history is scanned: a position applies its token's penalty if it
// is the token's first occurrence, with the count of the positions after
// it (quadratic in the history length); a longer one is counted in an LDS
// hash table (open addressing, linear probing, integer atomic counts), whose
// slots then apply one penalty per distinct token.  The counts are the same
// either way, and each distinct token is written by exactly one thread.  The arithmetic is fp32, one rounding per
// operation, in the documented order (the library is built without
// floating-point contraction and with a correctly rounded divide).

#include "penalty_dev.h"

namespace {

constexpr int THREADS = 256;
constexpr int HASH_MIN = 128;  // longer histories of dense rows are counted in a hash table
constexpr int TABLE_BITS = 13;
constexpr int TABLE = 1 << TABLE_BITS;  // hash slots: at least twice the longest history
static_assert(TABLE >= 2 * VS_MAX_WINDOW, "the table never fills");
constexpr size_t TABLE_BYTES = 2 * TABLE * sizeof(int32_t);  // keys, then counts

__global__ void __launch_bounds__(THREADS)
penalize_kernel(float* __restrict__ logits, const int32_t* __restrict__ ids, int64_t ld, int width,
                int vocab, const int32_t* __restrict__ ctx, int ctx_len,
                const int32_t* __restrict__ drafts, int n_drafts,
                bool tree, const int32_t* __restrict__ parent, int window, float rep,
                float pres, float freq) {
  __shared__ int32_t hist[VS_MAX_WINDOW];
  extern __shared__ int32_t table[];  // TABLE_BYTES when a dense row's history may exceed HASH_MIN
  __shared__ int32_t path[VS_MAX_DRAFTS + 1];
  __shared__ int path_len;
  const int row = blockIdx.x;
  // the draft tokens this row sees after the context: a chain's first
  // min(row, n_drafts) drafts, or a tree node's root path
  int nd = row < n_drafts ? row : n_drafts;
  const int32_t* dsrc = drafts;
  if (tree) {  // row 0 is the root; rows 1.. read tokens and parent
    if (threadIdx.x == 0) {
      int len = 0;
      if (row > 0) {
        // walk up from node row - 1; indices strictly decrease, so <= row steps
        int child = row - 1, q = parent[child];
        len = 1;
        while (q > -1 && q < child) {
          ++len;
          child = q;
          q = parent[q];
        }
        child = row - 1;
        for (int i = len - 1; i >= 0; --i) {
          path[i] = drafts[child];
          child = parent[child];
        }
      }
      path_len = len;
    }
    __syncthreads();
    nd = path_len;
    dsrc = path;
  }
  const int64_t total = static_cast<int64_t>(ctx_len) + nd;
  const int hlen = static_cast<int>(total < window ? total : window);
  const int64_t start = total - hlen;  // position of H_i[0] in ctx || drafts
  for (int j = threadIdx.x; j < hlen; j += blockDim.x) {
    const int64_t pos = start + j;
    int32_t t = pos < ctx_len ? ctx[pos] : dsrc[pos - ctx_len];
    hist[j] = (t >= 0 && t < vocab) ? t : -1;  // ids outside the vocabulary never match
  }
  __syncthreads();

  float* lrow = logits + static_cast<int64_t>(row) * ld;
  if (ids == nullptr && hlen > HASH_MIN) {  // uniform; the launch provides the table
    int32_t* key = table;
    int32_t* cnt = table + TABLE;
    for (int q = threadIdx.x; q < TABLE; q += blockDim.x) {
      key[q] = -1;
      cnt[q] = 0;
    }
    __syncthreads();
    for (int j = threadIdx.x; j < hlen; j += blockDim.x) {
      const int32_t t = hist[j];
      if (t < 0) continue;
      uint32_t q = (static_cast<uint32_t>(t) * 2654435761u) >> (32 - TABLE_BITS);
      // at most hlen <= TABLE / 2 distinct keys: an empty slot is always found
      for (;;) {
        const int32_t prev = atomicCAS(&key[q], -1, t);
        if (prev == -1 || prev == t) break;
        q = (q + 1) & (TABLE - 1);
      }
      atomicAdd(&cnt[q], 1);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < TABLE; q += blockDim.x) {
      const int32_t t = key[q];
      if (t >= 0) lrow[t] = penalize_one(lrow[t], cnt[q], rep, pres, freq);
    }
    return;
  }
  if (ids == nullptr) {
    for (int j = threadIdx.x; j < hlen; j += blockDim.x) {
      const int32_t t = hist[j];
      if (t < 0) continue;
      bool first = true;
      for (int i = 0; i < j && first; ++i) first = hist[i] != t;
      if (!first) continue;
      int c = 1;
      for (int i = j + 1; i < hlen; ++i) c += hist[i] == t;
      lrow[t] = penalize_one(lrow[t], c, rep, pres, freq);
    }
  } else {
    __shared__ int part[THREADS];  // per-thread counts of the current chunk
    const int32_t* irow = ids + static_cast<int64_t>(row) * ld;
    for (int base = 0; base < width; base += THREADS) {  // uniform trip count
      const int nslot = width - base < THREADS ? width - base : THREADS;
      const int tps = THREADS / nslot;  // threads per slot; nslot * tps <= THREADS
      const int slot = threadIdx.x / tps;
      int c = 0;
      if (slot < nslot) {
        const int32_t t = irow[base + slot];
        if (t >= 0 && t < vocab)
          for (int i = threadIdx.x % tps; i < hlen; i += tps) c += hist[i] == t;
      }
      part[threadIdx.x] = c;
      __syncthreads();
      if (threadIdx.x < nslot) {
        int total = 0;
        for (int j = 0; j < tps; ++j) total += part[threadIdx.x * tps + j];
        float* l = lrow + base + threadIdx.x;
        if (total > 0) *l = penalize_one(*l, total, rep, pres, freq);
      }
      __syncthreads();  // part is reused by the next chunk
    }
  }
}

}  // namespace

extern "C" int penalize_rows(float* logits, const int32_t* ids, int64_t ld, int rows, int width,
                             int vocab, const int32_t* ctx, int ctx_len, const int32_t* drafts,
                             int n_drafts, int window, float repeat, float presence,
                             float frequency, hipStream_t stream) {
  if (!logits) return VS_ERR_NULL;
  if (ctx_len < 0 || n_drafts < 0) return VS_ERR_SHAPE;
  if ((ctx_len > 0 && !ctx) || (n_drafts > 0 && !drafts)) return VS_ERR_NULL;
  if (rows < 1 || rows > 4096 || width < 1 || ld < width || vocab < 1) return VS_ERR_SHAPE;
  if (ids == nullptr && width != vocab) return VS_ERR_SHAPE;
  if (window < 0 || window > VS_MAX_WINDOW) return VS_ERR_PARAM;
  if (!(repeat > 0.f) || !__builtin_isfinite(repeat) || !__builtin_isfinite(presence) ||
      !__builtin_isfinite(frequency))
    return VS_ERR_PARAM;
  if (window == 0 || (ctx_len == 0 && n_drafts == 0)) return VS_OK;  // nothing to penalise
  // no row's history is longer than min(window, ctx_len + n_drafts)
  const size_t shm = ids == nullptr && window > HASH_MIN &&
                             static_cast<int64_t>(ctx_len) + n_drafts > HASH_MIN
                         ? TABLE_BYTES
                         : 0;
  penalize_kernel<<<dim3(rows), dim3(THREADS), shm, stream>>>(logits, ids, ld, width, vocab, ctx,
                                                              ctx_len, drafts, n_drafts, false,
                                                              nullptr, window, repeat, presence,
                                                              frequency);
  return vs::check_launch();
}

extern "C" int penalize_tree_rows(float* logits, const int32_t* ids, int64_t ld, int width,
                                  int vocab, const int32_t* ctx, int ctx_len,
                                  const int32_t* tokens, const int32_t* parent, int n_nodes,
                                  int window, float repeat, float presence, float frequency,
                                  hipStream_t stream) {
  if (!logits) return VS_ERR_NULL;
  if (ctx_len < 0 || n_nodes < 0 || n_nodes > VS_MAX_DRAFTS) return VS_ERR_SHAPE;
  if ((ctx_len > 0 && !ctx) || (n_nodes > 0 && (!tokens || !parent))) return VS_ERR_NULL;
  if (width < 1 || ld < width || vocab < 1) return VS_ERR_SHAPE;
  if (ids == nullptr && width != vocab) return VS_ERR_SHAPE;
  if (window < 0 || window > VS_MAX_WINDOW) return VS_ERR_PARAM;
  if (!(repeat > 0.f) || !__builtin_isfinite(repeat) || !__builtin_isfinite(presence) ||
      !__builtin_isfinite(frequency))
    return VS_ERR_PARAM;
  if (window == 0 || (ctx_len == 0 && n_nodes == 0)) return VS_OK;  // nothing to penalise
  // a node's path holds at most n_nodes tokens
  const size_t shm = ids == nullptr && window > HASH_MIN &&
                             static_cast<int64_t>(ctx_len) + n_nodes > HASH_MIN
                         ? TABLE_BYTES
                         : 0;
  penalize_kernel<<<dim3(n_nodes + 1), dim3(THREADS), shm, stream>>>(
      logits, ids, ld, width, vocab, ctx, ctx_len, tokens, n_nodes, true, parent, window, repeat,
      presence, frequency);
  return vs::check_launch();
}
