// topk_rows: per-row top-K (K <= 64) in the sampler's pool order.
//
// "Speculative decoding on RDNA", §03: the sampler's 64-wide pool and its tie
// order.  "feat(dflash): developer-only online draft tuning", "Code map": a
// one-block-per-row top-K ate the speculative gain; several workgroups per
// row fix it, and the result must be byte-identical with ties, NaN and -inf.
//
// Each element becomes a unique 64-bit key (value order, then complemented
// index; see vs_internal.h), so "top-K" is "the K largest keys" and there
// are no ties left to break.  Every kernel is one wavefront per unit of work
// (no workgroup barriers), and every selection is a threshold filter: a
// value every top-K element must reach, the few elements that reach it, and
// their ranks among themselves.  Two launches:
//   chunk stage: per (row, chunk), the K largest keys of the chunk (see
//                topk_chunk_kernel); rows of several chunks write them
//                sorted to the workspace.  Chunks hold 4096 elements for
//                batches and 1024 for a handful of rows, so that a single
//                verify window still spreads over the whole chip;
//   merge stage: per row, the K largest of the chunks' K candidates (see
//                topk_merge_kernel), written as values (the input's bits)
//                and indices.
// A row of one chunk is finished by the chunk stage alone.  Both stages fall
// back to an exact radix select when adversarial ties leave too many
// survivors.  The selection is exact integer work, so the result does not
// depend on scheduling or on the chunking.

#include <atomic>
#include <mutex>

#include "topk_dev.h"

namespace {

template <int NPL, int GROUPS>
__global__ void __launch_bounds__(64 * WAVES)
topk_chunk_kernel(const float* __restrict__ X, int64_t ldx, int rows, int V, int K, int chunks,
                  uint64_t* __restrict__ ws, float* __restrict__ out_vals,
                  int32_t* __restrict__ out_idx, int64_t ld_out) {
  __shared__ WaveShared shared[WAVES];
  const int w = vs::wave_index();
  // rows * chunks < 2^30 (rows <= 2^24, chunks <= 64 for many rows): 32-bit
  // scalar arithmetic
  const uint32_t unit = blockIdx.x * WAVES + static_cast<uint32_t>(w);
  if (unit >= static_cast<uint32_t>(rows) * static_cast<uint32_t>(chunks)) return;  // whole wave; no block barriers
  const int row = chunks == 1 ? static_cast<int>(unit) : static_cast<int>(unit / static_cast<uint32_t>(chunks));
  const int chunk = static_cast<int>(unit - static_cast<uint32_t>(row) * static_cast<uint32_t>(chunks));
  chunk_unit<NPL, GROUPS, false>(shared[w], X, ldx, row, chunk, V, K, chunks, ws, out_vals, out_idx, ld_out,
                                 NoPre{});
}

__global__ void __launch_bounds__(64 * WAVES)
topk_merge_kernel(const float* __restrict__ X, int64_t ldx, int rows, int V, int K, int chunks, int lg_jp,
                  int lg_j2, const uint64_t* __restrict__ ws, float* __restrict__ out_vals,
                  int32_t* __restrict__ out_idx, int64_t ld_out) {
  __shared__ MergeShared shared[WAVES];
  const int w = vs::wave_index();
  const int row = blockIdx.x * WAVES + w;
  if (row >= rows) return;  // whole wave; no block barriers
  merge_row(shared[w], X, ldx, row, V, K, chunks, lg_jp, lg_j2, ws, out_vals + static_cast<int64_t>(row) * ld_out,
            out_idx + static_cast<int64_t>(row) * ld_out);
}

}  // namespace

extern "C" size_t topk_rows_workspace_bytes(int rows, int V, int K) {
  if (rows < 1 || V < 1 || K < 1) return 0;
  const Plan p = plan_for(rows, V);
  if (p.chunks <= 1) return 0;
  return static_cast<size_t>(rows) * p.chunks * K * sizeof(uint64_t);
}

namespace {

// Both launches of a top-K call; ws holds topk_rows_workspace_bytes(rows, V,
// K) bytes (checked by the callers).
int launch_topk(const float* X, int64_t ldx, int rows, int V, int K, float* out_vals,
                int32_t* out_idx, int64_t ld_out, uint64_t* ws, hipStream_t stream) {
  const Plan p = plan_for(rows, V);
  static_assert(MAX_CHUNKS <= 256, "the merge's threshold entries fit four per lane");
  static_assert(MAX_CHUNKS * 4 <= 64 * MERGE_LOADS, "the merge reads at least four entries per chunk");
  const int64_t units = static_cast<int64_t>(rows) * p.chunks;
  const dim3 grid(static_cast<unsigned>((units + WAVES - 1) / WAVES)), block(64 * WAVES);
  if (p.small)
    topk_chunk_kernel<16, 4><<<grid, block, 0, stream>>>(X, ldx, rows, V, K, p.chunks, ws, out_vals,
                                                          out_idx, ld_out);
  else
    topk_chunk_kernel<64, 4><<<grid, block, 0, stream>>>(X, ldx, rows, V, K, p.chunks, ws, out_vals,
                                                          out_idx, ld_out);
  int st = vs::check_launch();
  if (st != VS_OK || p.chunks == 1) return st;
  int lg_jp, lg_j2;
  merge_reads(p.chunks, K, lg_jp, lg_j2);
  topk_merge_kernel<<<dim3(static_cast<unsigned>((rows + WAVES - 1) / WAVES)), block, 0, stream>>>(
      X, ldx, rows, V, K, p.chunks, lg_jp, lg_j2, ws, out_vals, out_idx, ld_out);
  return vs::check_launch();
}

int check_topk_args(const float* X, int64_t ldx, int rows, int V, int K, const float* out_vals,
                    const int32_t* out_idx, int64_t ld_out) {
  if (!X || !out_vals || !out_idx) return VS_ERR_NULL;
  if (rows < 1 || rows > (1 << 24) || K < 1 || K > VS_POOL || V < K || V > VS_MAX_VOCAB)
    return VS_ERR_SHAPE;
  if (ldx < V || ld_out < K) return VS_ERR_SHAPE;
  return VS_OK;
}

// The fixed scratch area of topk_rows_noalloc: one copy per GPU, in device
// memory for the life of the process.  Host code never uses this name as an
// address; it uses the per-device address that hipGetSymbolAddress returns.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t{4} << 20;
__device__ __align__(256) uint64_t scratch[NOALLOC_SCRATCH_BYTES / sizeof(uint64_t)];

constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_scratch_addr[MAX_DEVICES];
std::mutex g_scratch_mutex;

// The address of `scratch` on the current device, looked up once per device.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return vs::hip_status(e);
  if (dev < 0 || dev >= MAX_DEVICES) return VS_ERR_UNSUPPORTED;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return vs::hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol);
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return VS_OK;
}

}  // namespace

extern "C" int topk_rows(const float* X, int64_t ldx, int rows, int V, int K, float* out_vals,
                         int32_t* out_idx, int64_t ld_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  int st = check_topk_args(X, ldx, rows, V, K, out_vals, out_idx, ld_out);
  if (st != VS_OK) return st;
  const size_t need = topk_rows_workspace_bytes(rows, V, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return VS_ERR_WORKSPACE;
  if (need > 0 && !vs::aligned16(workspace)) return VS_ERR_ALIGN;
  return launch_topk(X, ldx, rows, V, K, out_vals, out_idx, ld_out, static_cast<uint64_t*>(workspace),
                     stream);
}

extern "C" size_t topk_rows_noalloc_max_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

extern "C" int topk_rows_noalloc(const float* X, int64_t ldx, int rows, int V, int K,
                                 float* out_vals, int32_t* out_idx, int64_t ld_out,
                                 hipStream_t stream) {
  int st = check_topk_args(X, ldx, rows, V, K, out_vals, out_idx, ld_out);
  if (st != VS_OK) return st;
  if (topk_rows_workspace_bytes(rows, V, K) > NOALLOC_SCRATCH_BYTES) return VS_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != VS_OK) return st;
  return launch_topk(X, ldx, rows, V, K, out_vals, out_idx, ld_out, static_cast<uint64_t*>(ws), stream);
}
