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
// 256*(j/4) + 4*l + j%4, so every load is a coalesced 1 KB), in four groups
// of 16.  Steps, each cheap in vector instructions:
//   1. the float maximum of each group (NaN is skipped or, if signalling,
//      makes the maximum NaN: either way the group holds an element at
//      least as large, in key order, as the maximum found);
//   2. v = the K-th largest value key of the 256 group maxima, by a bitwise
//      search on ballot counts.  The K groups at or above v hold K distinct
//      elements of value key >= v, so the top K are among the survivors
//      "value key >= v", a single float comparison x >= t for t the value
//      whose key is v (NaN never passes, -0 and +0 compare equal as their
//      keys do; fp32 denormals are kept, so the comparison is exact);
//   3. the survivors (about 73 for K = 64 on ordinary rows) are compacted to
//      LDS as (bits, chunk index) pairs;
//   4. each survivor's rank is the number of larger 64-bit keys among them;
//      ranks below K are the output positions.
// If fewer than K group maxima are real numbers, every valid element
// survives; if more than CAND survive (adversarial rows), an exact per-wave
// radix select on the 64-bit keys finds the K-th largest key and only the
// keys at or above it are compacted.  Either way the result is exact: keys
// are unique.

constexpr int WAVES = 4;               // wavefronts per workgroup
constexpr int NPL = CHUNK / 64;        // values per lane
constexpr int GROUPS = 4;              // group maxima per lane
constexpr int GL = NPL / GROUPS;       // values per group
constexpr int CAND = 256;              // survivors ranked directly

struct WaveShared {
  uint32_t bits[CAND + 1];  // survivors' input bits; slot CAND absorbs overflow writes
  uint32_t li[CAND + 1];    // survivors' chunk-local indices
  uint64_t key[CAND];       // survivors' 64-bit keys, zero-padded
  uint32_t hist[256];       // radix-select histogram (fallback only)
};

// Makes this wave's LDS writes visible to its other lanes before they read.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ int chunk_index(int lane, int j) { return ((j >> 2) << 8) + (lane << 2) + (j & 3); }

// The hardware three-way maximum, without the compiler's NaN quieting of
// each operand (its effect on NaN is covered by step 1 above).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// The float whose value key is v (v >= 1 and the key of a number).
__device__ __forceinline__ uint32_t key_bits(uint32_t v) { return (v & 0x80000000u) ? (v ^ 0x80000000u) : ~v; }

// Appends the elements of lane-column j that pass to the survivor list.
__device__ __forceinline__ void compact_one(WaveShared& sh, int& count, bool take, uint32_t bits, uint32_t li) {
  const uint64_t m = __ballot(take);
  if (m == 0) return;  // uniform
  if (take) {
    uint32_t slot = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                              __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), count));
    slot = slot < CAND ? slot : CAND;
    sh.bits[slot] = bits;
    sh.li[slot] = li;
  }
  count += __popcll(m);
}

// Ranks the c <= 64*E survivors and writes those of rank < K.
template <int E>
__device__ __forceinline__ void rank_and_write(WaveShared& sh, int c, int K, int base, int chunks,
                                               int64_t row, int chunk, uint64_t* __restrict__ ws,
                                               float* __restrict__ out_vals,
                                               int32_t* __restrict__ out_idx, int64_t ld_out) {
  const int lane = threadIdx.x & 63;
  uint32_t b[E], l[E];
  uint64_t k[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int s = lane + 64 * r;
    const bool live = s < c;
    b[r] = live ? sh.bits[s] : 0u;
    l[r] = live ? sh.li[s] : 0u;
    k[r] = live ? ((static_cast<uint64_t>(vs::value_key(b[r])) << 32) |
                   static_cast<uint32_t>(~static_cast<uint32_t>(base + static_cast<int>(l[r]))))
                : 0ull;
    sh.key[s] = k[r];  // empty slots hold 0, which is below every key
  }
  wave_lds_sync();
  int rank[E];
#pragma unroll
  for (int r = 0; r < E; ++r) rank[r] = 0;
  const int cr = (c + 3) & ~3;  // <= 64*E; keys past c are 0
  for (int s = 0; s < cr; s += 4) {
    const uint64_t k0 = sh.key[s], k1 = sh.key[s + 1], k2 = sh.key[s + 2], k3 = sh.key[s + 3];
#pragma unroll
    for (int r = 0; r < E; ++r)
      rank[r] += (k0 > k[r]) + (k1 > k[r]) + (k2 > k[r]) + (k3 > k[r]);
  }
  const bool single = chunks == 1;
  int64_t obase = single ? row * ld_out : (row * chunks + chunk) * K;
#pragma unroll
  for (int r = 0; r < E; ++r) {
    if (lane + 64 * r < c && rank[r] < K) {
      if (single) {
        out_idx[obase + rank[r]] = base + static_cast<int>(l[r]);
        out_vals[obase + rank[r]] = __builtin_bit_cast(float, b[r]);  // the input's bits
      } else {
        ws[obase + rank[r]] = k[r];
      }
    }
  }
  if (lane >= c && lane < K) {  // fewer than K elements: empty entries
    if (single) {
      out_idx[obase + lane] = -1;
      out_vals[obase + lane] = __builtin_nanf("");
    } else {
      ws[obase + lane] = 0ull;
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

  // the lane's 64 values; elements past the row's end read as NaN, which no
  // maximum or threshold comparison selects
  float x[NPL];
  const bool vec = n == CHUNK && ((reinterpret_cast<uintptr_t>(xrow + base) & 15u) == 0);
  if (vec) {
#pragma unroll
    for (int q = 0; q < NPL / 4; ++q) {
      const float4 f = *reinterpret_cast<const float4*>(xrow + base + (q << 8) + (lane << 2));
      x[4 * q + 0] = f.x;
      x[4 * q + 1] = f.y;
      x[4 * q + 2] = f.z;
      x[4 * q + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int li = chunk_index(lane, j);
      x[j] = li < n ? xrow[base + li] : __builtin_nanf("");
    }
  }

  // 1-2: group maxima and the K-th largest of their value keys
  uint32_t mk[GROUPS];
#pragma unroll
  for (int g = 0; g < GROUPS; ++g) {
    float m = max3f(x[GL * g], x[GL * g + 1], x[GL * g + 2]);
#pragma unroll
    for (int i = 3; i + 1 < GL; i += 2) m = max3f(m, x[GL * g + i], x[GL * g + i + 1]);
    if ((GL - 3) % 2) m = max3f(m, x[GL * g + GL - 1], x[GL * g + GL - 1]);
    mk[g] = vs::value_key(__builtin_bit_cast(uint32_t, m));
  }
  uint32_t v = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = v | (1u << bit);
    int c = 0;
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) c += __popcll(__ballot(mk[g] >= cand));
    if (c >= K) v = cand;
  }

  // 3: compaction
  const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
  int count = 0;
  if (v != 0) {
    const float t = __builtin_bit_cast(float, key_bits(v));
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      compact_one(sh, count, x[j] >= t, __builtin_bit_cast(uint32_t, x[j]),
                  lane4 | static_cast<uint32_t>(((j >> 2) << 8) | (j & 3)));
  } else {  // fewer than K group maxima are numbers: every valid element
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int li = chunk_index(lane, j);
      compact_one(sh, count, li < n, __builtin_bit_cast(uint32_t, x[j]), static_cast<uint32_t>(li));
    }
  }

  if (count > CAND) {
    // exact radix select of the K-th largest key, 8 bits at a time (more
    // than CAND >= K valid keys exist here).  This path is rare (adversarial
    // rows); it re-reads the chunk each pass so that its keys never occupy
    // registers alongside the main path's.
    uint64_t prefix = 0;
    int need = K;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      const uint64_t hmask = pass == 0 ? 0ull : (~0ull << (shift + 8));
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) sh.hist[4 * lane + bb] = 0u;
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
      for (int bb = 0; bb < 4; ++bb) c[bb] = sh.hist[255 - 4 * lane - bb];
      const uint32_t sum = c[0] + c[1] + c[2] + c[3];
      uint32_t incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      const uint32_t excl = incl - sum;
      const bool mine = excl < static_cast<uint32_t>(need) && static_cast<uint32_t>(need) <= incl;
      int digit = 0, rest = 0;
      if (mine) {
        uint32_t cum = excl;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          if (cum + c[bb] >= static_cast<uint32_t>(need)) {
            digit = 255 - 4 * lane - bb;
            rest = need - static_cast<int>(cum);
            break;
          }
          cum += c[bb];
        }
      }
      const int src = __ffsll(static_cast<long long>(__ballot(mine))) - 1;
      digit = vs::bcast(digit, src);
      need = vs::bcast(rest, src);
      prefix |= static_cast<uint64_t>(digit) << shift;
      wave_lds_sync();
    }
    // exactly K keys are >= prefix: compact them again
    count = 0;
    asm volatile("" ::: "memory");
    for (int j = 0; j < NPL; ++j) {
      const int li = chunk_index(lane, j);
      uint32_t bits = 0;
      uint64_t kj = 0;
      if (li < n) {
        bits = __builtin_bit_cast(uint32_t, xrow[base + li]);
        kj = (static_cast<uint64_t>(vs::value_key(bits)) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(base + li));
      }
      compact_one(sh, count, kj != 0 && kj >= prefix, bits, static_cast<uint32_t>(li));
    }
  }

  // 4: ranks and output
  wave_lds_sync();
  if (count <= 64)
    rank_and_write<1>(sh, count, K, base, chunks, row, chunk, ws, out_vals, out_idx, ld_out);
  else if (count <= 128)
    rank_and_write<2>(sh, count, K, base, chunks, row, chunk, ws, out_vals, out_idx, ld_out);
  else
    rank_and_write<4>(sh, count, K, base, chunks, row, chunk, ws, out_vals, out_idx, ld_out);
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
