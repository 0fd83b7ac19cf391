// topk_rows: per-row top-K (K <= 64) in the sampler's pool order.
//
// "Speculative decoding on RDNA", §03: the sampler's 64-wide pool and its tie
// order.  "feat(dflash): developer-only online draft tuning", "Code map": a
// one-block-per-row top-K ate the speculative gain; several workgroups per
// row fix it, and the result must be byte-identical with ties, NaN and -inf.
//
// Each element becomes a unique 64-bit key (value order, then complemented
// index; see vs_internal.h), so "top-K" is "the K largest keys" and there
// are no ties left to break.  Two launches:
//   stage 1: one workgroup per (row, chunk); each 256-thread workgroup radix-selects the
//            K largest keys of a 4096-element chunk (eight 8-bit digit
//            passes over LDS histograms) and writes them, sorted, to the
//            workspace;
//   stage 2: one workgroup per row selects the K largest of the chunks' K
//            candidates the same way and writes values (the input's bits,
//            re-read by index) and indices.
// A row of at most one chunk is finished by stage 1 alone.  The selection is
// exact integer work, so the result does not depend on scheduling.

#include "vs_internal.h"

namespace {

constexpr int THREADS = 256;
constexpr int CHUNK = 4096;
constexpr int PER = CHUNK / THREADS;  // keys per thread
constexpr int MAX_CHUNKS = VS_MAX_VOCAB / CHUNK;

struct SelectShared {
  uint32_t hist[256];
  uint64_t sel[VS_POOL];
  uint64_t prefix;
  int need;
  int count;
};

// Leaves the K largest keys of the block (keys of 0 are empty slots) in
// sh.sel[0, K), sorted descending, padded with 0.  All threads must call it.
__device__ void block_topk(const uint64_t (&key)[PER], int K, SelectShared& sh) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  if (tid == 0) sh.count = 0;
  __syncthreads();
  int mine = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) mine += key[e] != 0;
  if (mine) atomicAdd(&sh.count, mine);
  __syncthreads();
  const int n_real = sh.count;
  __syncthreads();  // every thread has read the count before it is reused

  uint64_t thr = 1;  // every real key is >= 1
  if (n_real > K) {
    uint64_t prefix = 0;
    int need = K;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      const uint64_t hmask = pass == 0 ? 0ull : (~0ull << (shift + 8));
      sh.hist[tid] = 0;  // THREADS == 256 bins
      __syncthreads();
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const uint64_t k = key[e];
        if (k != 0 && ((k ^ prefix) & hmask) == 0)
          atomicAdd(&sh.hist[static_cast<uint32_t>(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l covers bins 255-4l .. 252-4l, highest first
        uint32_t c[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) c[b] = sh.hist[255 - 4 * lane - b];
        const uint32_t s = c[0] + c[1] + c[2] + c[3];
        uint32_t incl = s;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t v = __shfl_up(incl, off, 64);
          if (lane >= off) incl += v;
        }
        const uint32_t excl = incl - s;
        if (excl < static_cast<uint32_t>(need) && static_cast<uint32_t>(need) <= incl) {
          uint32_t cum = excl;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            if (cum + c[b] >= static_cast<uint32_t>(need)) {
              const uint64_t digit = static_cast<uint64_t>(255 - 4 * lane - b);
              sh.prefix = prefix | (digit << shift);
              sh.need = need - static_cast<int>(cum);
              break;
            }
            cum += c[b];
          }
        }
      }
      __syncthreads();
      prefix = sh.prefix;
      need = sh.need;
      __syncthreads();
    }
    thr = prefix;  // the K-th largest key; keys are unique, so exactly K are >= thr
  }

  if (tid == 0) sh.count = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (key[e] != 0 && key[e] >= thr) {
      const int slot = atomicAdd(&sh.count, 1);
      if (slot < VS_POOL) sh.sel[slot] = key[e];  // exactly K <= VS_POOL keys qualify
    }
  }
  __syncthreads();
  if (tid < 64) {
    uint64_t k = lane < sh.count ? sh.sel[lane] : 0ull;
    uint32_t dummy = 0;
    vs::wave_sort_desc(k, dummy);
    sh.sel[lane] = k;
  }
  __syncthreads();
}

__device__ __forceinline__ void write_row(const float* __restrict__ xrow, const uint64_t* sel,
                                          int K, float* __restrict__ out_vals,
                                          int32_t* __restrict__ out_idx) {
  const int lane = threadIdx.x;
  if (lane < K) {
    const uint32_t idx = vs::key_index(sel[lane]);
    out_idx[lane] = static_cast<int32_t>(idx);
    out_vals[lane] = xrow[idx];  // the input's bits, unchanged
  }
}

__global__ void __launch_bounds__(THREADS)
topk_stage1(const float* __restrict__ X, int64_t ldx, int V, int K, int chunks,
            uint64_t* __restrict__ ws, float* __restrict__ out_vals, int32_t* __restrict__ out_idx,
            int64_t ld_out) {
  __shared__ SelectShared sh;
  const int row = blockIdx.x / chunks, chunk = blockIdx.x % chunks;
  const float* xrow = X + static_cast<int64_t>(row) * ldx;
  const int base = chunk * CHUNK;
  uint64_t key[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int idx = base + e * THREADS + threadIdx.x;
    key[e] = idx < V ? vs::order_key(__builtin_bit_cast(uint32_t, xrow[idx]), static_cast<uint32_t>(idx))
                     : 0ull;
  }
  block_topk(key, K, sh);
  if (chunks == 1) {
    write_row(xrow, sh.sel, K, out_vals + static_cast<int64_t>(row) * ld_out,
              out_idx + static_cast<int64_t>(row) * ld_out);
  } else if (threadIdx.x < K) {
    ws[(static_cast<int64_t>(row) * chunks + chunk) * K + threadIdx.x] = sh.sel[threadIdx.x];
  }
}

__global__ void __launch_bounds__(THREADS)
topk_stage2(const float* __restrict__ X, int64_t ldx, int K, int chunks,
            const uint64_t* __restrict__ ws, float* __restrict__ out_vals,
            int32_t* __restrict__ out_idx, int64_t ld_out) {
  __shared__ SelectShared sh;
  const int row = blockIdx.x;
  const int n = chunks * K;  // <= MAX_CHUNKS * VS_POOL == CHUNK
  const uint64_t* src = ws + static_cast<int64_t>(row) * n;
  uint64_t key[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = e * THREADS + threadIdx.x;
    key[e] = c < n ? src[c] : 0ull;
  }
  block_topk(key, K, sh);
  write_row(X + static_cast<int64_t>(row) * ldx, sh.sel, K,
            out_vals + static_cast<int64_t>(row) * ld_out, out_idx + static_cast<int64_t>(row) * ld_out);
}

int n_chunks(int V) { return (V + CHUNK - 1) / CHUNK; }

}  // namespace

extern "C" size_t topk_rows_workspace_bytes(int rows, int V, int K) {
  if (rows < 1 || V < 1 || K < 1) return 0;
  const int chunks = n_chunks(V);
  if (chunks <= 1) return 0;
  return static_cast<size_t>(rows) * chunks * K * sizeof(uint64_t);
}

extern "C" int topk_rows(const float* X, int64_t ldx, int rows, int V, int K, float* out_vals,
                         int32_t* out_idx, int64_t ld_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (!X || !out_vals || !out_idx) return VS_ERR_NULL;
  if (rows < 1 || rows > (1 << 24) || K < 1 || K > VS_POOL || V < K || V > VS_MAX_VOCAB)
    return VS_ERR_SHAPE;
  if (ldx < V || ld_out < K) return VS_ERR_SHAPE;
  const int chunks = n_chunks(V);
  static_assert(MAX_CHUNKS * VS_POOL <= CHUNK, "stage 2 holds all candidates of a row");
  const size_t need = topk_rows_workspace_bytes(rows, V, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return VS_ERR_WORKSPACE;
  if (need > 0 && !vs::aligned16(workspace)) return VS_ERR_ALIGN;
  uint64_t* ws = static_cast<uint64_t*>(workspace);
  topk_stage1<<<dim3(chunks * rows), dim3(THREADS), 0, stream>>>(X, ldx, V, K, chunks, ws, out_vals,
                                                                out_idx, ld_out);
  int st = vs::check_launch();
  if (st != VS_OK || chunks == 1) return st;
  topk_stage2<<<dim3(rows), dim3(THREADS), 0, stream>>>(X, ldx, K, chunks, ws, out_vals, out_idx,
                                                        ld_out);
  return vs::check_launch();
}
