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
//   stage 1: per (row, chunk of 4096 elements), the K largest keys of the
//            chunk: a 256-thread radix select for small batches, one
//            wavefront with a threshold filter for large ones (see
//            topk_wave_stage1); rows of several chunks write them sorted to
//            the workspace;
//   stage 2: one workgroup per row selects the K largest of the chunks' K
//            candidates by radix select (eight 8-bit digit passes over LDS
//            histograms) and writes values (the input's bits, re-read by
//            index) and indices.
// A row of at most one chunk is finished by stage 1 alone.  The selection is
// exact integer work, so the result does not depend on scheduling.

#include "wave_ops.h"

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

// Stage 1, one 256-thread workgroup per (row, chunk): lower latency when there
// are few chunks in total (one verify window), so the chip is mostly idle.
__global__ void __launch_bounds__(THREADS)
topk_block_stage1(const float* __restrict__ X, int64_t ldx, int V, int K, int chunks,
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

// ---------------------------------------------------------------------------
// Stage 1, one wavefront per (row, chunk of up to 4096 elements).
//
// Lane l holds 64 values of the chunk (element j of the lane is chunk index
// 256*(j/4) + 4*l + j%4, so every load is a coalesced 1 KB).  The K-th
// largest of 128 group maxima (32 keys each) is a threshold at least K keys
// reach (the maxima are distinct keys), so only the keys at or above it can
// be in the top K.  For ordinary rows they number about ninety; they
// are compacted to LDS and bitonic-sorted across the wave, and the first K
// are the answer.  If more than CAND survive (adversarial rows), an exact
// per-wave radix select on the 64-bit keys finds the K-th largest key
// instead.  Either way the result is exact: keys are unique.

constexpr int WAVES = 4;               // wavefronts per workgroup
constexpr int NPL = CHUNK / 64;        // values per lane
constexpr int GROUPS = 2;              // group maxima per lane for the threshold
constexpr int CAND = 64 * GROUPS;      // candidates sorted directly (GROUPS per lane)

struct WaveShared {
  uint64_t cand[CAND];
  uint32_t hist[256];
};

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m, 64);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v & 0xffffffffu), src));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), src));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Makes this wave's LDS writes visible to its other lanes before they read.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ int chunk_index(int lane, int j) { return ((j >> 2) << 8) + (lane << 2) + (j & 3); }

// Sorts 64*E keys held E per lane (element E*lane + r) in descending order.
template <int E>
__device__ __forceinline__ void wave_sort_desc_n(uint64_t (&k)[E]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64 * E; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= E) {
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const uint64_t other = shfl_xor64(k[r], stride / E);
          const int e = E * lane + r;
          const bool desc = (e & size) == 0;
          const bool lower = (e & stride) == 0;
          const bool take_max = lower == desc;
          k[r] = take_max ? (other > k[r] ? other : k[r]) : (other < k[r] ? other : k[r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < E; ++r) {
          if (r & stride) continue;
          const int r2 = r | stride;
          const int e = E * lane + r;
          const bool desc = (e & size) == 0;
          const uint64_t a = k[r], b = k[r2];
          const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
          k[r] = desc ? hi : lo;
          k[r2] = desc ? lo : hi;
        }
      }
    }
  }
}

__global__ void __launch_bounds__(64 * WAVES)
topk_wave_stage1(const float* __restrict__ X, int64_t ldx, int rows, int V, int K, int chunks,
                 uint64_t* __restrict__ ws, float* __restrict__ out_vals,
                 int32_t* __restrict__ out_idx, int64_t ld_out) {
  __shared__ WaveShared shared[WAVES];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * WAVES + w;
  if (unit >= static_cast<int64_t>(rows) * chunks) return;  // whole wave; no block barriers
  const int row = static_cast<int>(unit / chunks);
  const int chunk = static_cast<int>(unit - static_cast<int64_t>(row) * chunks);
  WaveShared& sh = shared[w];
  const float* xrow = X + static_cast<int64_t>(row) * ldx;
  const int base = chunk * CHUNK;
  const int n = V - base < CHUNK ? V - base : CHUNK;

  // value keys of the lane's 64 elements (0 for elements past the row's end)
  uint32_t vk[NPL];
  const bool vec = n == CHUNK && ((reinterpret_cast<uintptr_t>(xrow + base) & 15u) == 0);
  if (vec) {
#pragma unroll
    for (int q = 0; q < NPL / 4; ++q) {
      const float4 f = *reinterpret_cast<const float4*>(xrow + base + (q << 8) + (lane << 2));
      vk[4 * q + 0] = vs::value_key(__builtin_bit_cast(uint32_t, f.x));
      vk[4 * q + 1] = vs::value_key(__builtin_bit_cast(uint32_t, f.y));
      vk[4 * q + 2] = vs::value_key(__builtin_bit_cast(uint32_t, f.z));
      vk[4 * q + 3] = vs::value_key(__builtin_bit_cast(uint32_t, f.w));
    }
  } else {
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int li = chunk_index(lane, j);
      vk[j] = li < n ? vs::value_key(__builtin_bit_cast(uint32_t, xrow[base + li])) : 0u;
    }
  }
  auto key = [&](int j) -> uint64_t {
    const int li = chunk_index(lane, j);
    return li < n ? ((static_cast<uint64_t>(vk[j]) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(base + li)))
                  : 0ull;
  };

  // threshold: the K-th largest of the 64*GROUPS group maxima (each lane's 64
  // keys in GROUPS runs); the K largest group maxima are K distinct keys.
  // Within a lane the index grows with j, so the first maximal value key in
  // a group has the largest complemented index.
  constexpr int GL = NPL / GROUPS;
  uint64_t gmax[GROUPS];
#pragma unroll
  for (int gi = 0; gi < GROUPS; ++gi) {
    uint32_t best = 0;
    int bj = -1;
#pragma unroll
    for (int j = GL * gi; j < GL * gi + GL; ++j) {
      const bool valid = chunk_index(lane, j) < n;
      if (valid && (bj < 0 || vk[j] > best)) {
        best = vk[j];
        bj = j;
      }
    }
    gmax[gi] = bj < 0 ? 0ull
                      : ((static_cast<uint64_t>(best) << 32) |
                         static_cast<uint32_t>(~static_cast<uint32_t>(base + chunk_index(lane, bj))));
  }
  wave_sort_desc_n<GROUPS>(gmax);
  // element K-1 of the sorted maxima sits in lane (K-1)/GROUPS, slot (K-1)%GROUPS
  uint64_t mine = gmax[0];
#pragma unroll
  for (int r = 1; r < GROUPS; ++r) mine = ((K - 1) % GROUPS) == r ? gmax[r] : mine;
  uint64_t thr = shfl64(mine, (K - 1) / GROUPS);
  if (thr == 0) thr = 1;  // fewer than K real keys: take them all

  // key(j) >= thr without forming the 64-bit key
  auto at_least = [&](int j, uint64_t t) -> bool {
    const uint32_t th = static_cast<uint32_t>(t >> 32), tl = static_cast<uint32_t>(t);
    const int li = chunk_index(lane, j);
    const uint32_t lo = static_cast<uint32_t>(~static_cast<uint32_t>(base + li));
    return li < n && (vk[j] > th || (vk[j] == th && lo >= tl));
  };
  // compact the keys >= thr to LDS while counting them (at most CAND kept)
  int count = 0;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const bool take = at_least(j, thr);
    const uint64_t m = __ballot(take);
    if (take) {
      const int slot = count + vs::lanes_below(m);
      if (slot < CAND) sh.cand[slot] = key(j);
    }
    count += __popcll(m);
  }

  if (count > CAND) {
    // exact radix select of the K-th largest key, 8 bits at a time.  This
    // path is rare (adversarial rows); it re-reads the chunk each pass so that
    // its keys never occupy registers alongside the main path's.
    uint64_t prefix = 0;
    int need = K;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      const uint64_t hmask = pass == 0 ? 0ull : (~0ull << (shift + 8));
#pragma unroll
      for (int b = 0; b < 4; ++b) sh.hist[4 * lane + b] = 0u;
      wave_lds_sync();
      asm volatile("" ::: "memory");  // keep the re-reads inside this pass
      for (int j = 0; j < NPL; ++j) {
        const int li = chunk_index(lane, j);
        if (li >= n) continue;
        const uint64_t kj = (static_cast<uint64_t>(vs::value_key(__builtin_bit_cast(uint32_t, xrow[base + li]))) << 32) |
                            static_cast<uint32_t>(~static_cast<uint32_t>(base + li));
        if (((kj ^ prefix) & hmask) == 0)
          atomicAdd(&sh.hist[static_cast<uint32_t>(kj >> shift) & 255u], 1u);
      }
      wave_lds_sync();
      uint32_t c[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) c[b] = sh.hist[255 - 4 * lane - b];
      const uint32_t sum = c[0] + c[1] + c[2] + c[3];
      uint32_t incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
      }
      const uint32_t excl = incl - sum;
      const bool mine = excl < static_cast<uint32_t>(need) && static_cast<uint32_t>(need) <= incl;
      int digit = 0, rest = 0;
      if (mine) {
        uint32_t cum = excl;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (cum + c[b] >= static_cast<uint32_t>(need)) {
            digit = 255 - 4 * lane - b;
            rest = need - static_cast<int>(cum);
            break;
          }
          cum += c[b];
        }
      }
      const int src = __ffsll(static_cast<long long>(__ballot(mine))) - 1;
      digit = vs::bcast(digit, src);
      need = vs::bcast(rest, src);
      prefix |= static_cast<uint64_t>(digit) << shift;
      wave_lds_sync();
    }
    thr = prefix;  // exactly K keys are >= thr: compact them again
    count = 0;
    asm volatile("" ::: "memory");
    for (int j = 0; j < NPL; ++j) {
      const int li = chunk_index(lane, j);
      uint64_t kj = 0;
      if (li < n)
        kj = (static_cast<uint64_t>(vs::value_key(__builtin_bit_cast(uint32_t, xrow[base + li]))) << 32) |
             static_cast<uint32_t>(~static_cast<uint32_t>(base + li));
      const bool take = kj != 0 && kj >= thr;
      const uint64_t m = __ballot(take);
      if (take) {
        const int slot = count + vs::lanes_below(m);
        if (slot < CAND) sh.cand[slot] = kj;
      }
      count += __popcll(m);
    }
  }
  const int pos = count;
  wave_lds_sync();
  uint64_t kc[GROUPS];
#pragma unroll
  for (int r = 0; r < GROUPS; ++r) {
    const int e = GROUPS * lane + r;
    kc[r] = e < pos && e < CAND ? sh.cand[e] : 0ull;
  }
  wave_lds_sync();
  wave_sort_desc_n<GROUPS>(kc);
#pragma unroll
  for (int r = 0; r < GROUPS; ++r) sh.cand[GROUPS * lane + r] = kc[r];
  wave_lds_sync();
  if (lane < K) {
    const uint64_t kk = sh.cand[lane];
    if (chunks == 1) {
      // a single-chunk row has V >= K real keys, so kk is never the empty key
      const uint32_t idx = vs::key_index(kk);
      const bool real = kk != 0;
      out_idx[static_cast<int64_t>(row) * ld_out + lane] = real ? static_cast<int32_t>(idx) : -1;
      out_vals[static_cast<int64_t>(row) * ld_out + lane] = real ? xrow[idx] : __builtin_nanf("");
    } else {
      ws[(static_cast<int64_t>(row) * chunks + chunk) * K + lane] = kk;
    }
  }
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
  // Both stage-1 kernels give the same keys: a workgroup per chunk has the
  // lower latency for a handful of rows, a wavefront per chunk the higher
  // throughput for batches.
  const int64_t units = static_cast<int64_t>(rows) * chunks;
  if (units < 2048) {
    topk_block_stage1<<<dim3(static_cast<unsigned>(units)), dim3(THREADS), 0, stream>>>(
        X, ldx, V, K, chunks, ws, out_vals, out_idx, ld_out);
  } else {
    topk_wave_stage1<<<dim3(static_cast<unsigned>((units + WAVES - 1) / WAVES)), dim3(64 * WAVES), 0,
                       stream>>>(X, ldx, rows, V, K, chunks, ws, out_vals, out_idx, ld_out);
  }
  int st = vs::check_launch();
  if (st != VS_OK || chunks == 1) return st;
  topk_stage2<<<dim3(rows), dim3(THREADS), 0, stream>>>(X, ldx, K, chunks, ws, out_vals, out_idx,
                                                        ld_out);
  return vs::check_launch();
}
