// Top-K in the sampler's pool order: the chunk stage and the merge stage as
// device functions of one 64-lane wave, and the chunking plan (see topk.hip
// for the design).
#pragma once

#include "wave_ops.h"

namespace {

constexpr int WAVES = 4;             // wavefronts per workgroup
constexpr int CAND = 256;            // survivors ranked directly
constexpr int SMALL_CHUNK = 1024;    // elements per chunk for a few rows
constexpr int LARGE_CHUNK = 4096;    // elements per chunk for batches
constexpr int MAX_CHUNKS = VS_MAX_VOCAB / SMALL_CHUNK;
constexpr int MERGE_LOADS = 24;      // candidates a merge lane reads in one round
constexpr int COARSE_BIT = 16;      // first threshold searches: low value-key bits searched only
constexpr int COARSE_SLACK = 8;     // while more than K + COARSE_SLACK keys are at or above
constexpr uint32_t NEG_INF_KEY = 0x007fffffu;  // value key of -inf, the smallest of a number
constexpr int SMALL_BATCH_UNITS = 2048;  // fewer 4096-chunks than this: small chunks

struct WaveShared {
  uint32_t bits[CAND + 1];  // survivors' input bits; slot CAND absorbs overflow writes
  uint32_t li[CAND + 1];    // survivors' chunk-local indices
  uint64_t key[CAND];       // survivors' 64-bit keys, zero-padded
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct MergeShared {
  uint64_t key[CAND + 1];     // survivors; slot CAND absorbs overflow writes
  uint32_t cont[MAX_CHUNKS];  // chunk lists: those to read on, the second round's
};

// Number of set bits of m in the lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m, uint32_t add = 0) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), add));
}

__device__ __forceinline__ int chunk_index(int lane, int j) { return ((j >> 2) << 8) + (lane << 2) + (j & 3); }

// The hardware three-way maximum, without the compiler's NaN quieting of
// each operand (its effect on NaN is covered by topk_chunk_kernel, step 1).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Keeps three ballots in distinct scalar registers until this point, so the
// compares that make them issue back to back instead of queueing on one
// condition register.
__device__ __forceinline__ void pin3(uint64_t a, uint64_t b, uint64_t c) { asm volatile("" ::"s"(a), "s"(b), "s"(c)); }
template <int N>
__device__ __forceinline__ void pin_ballots(const uint64_t (&b)[N]) {
  static_assert(N >= 1 && N <= 4, "ballots");
  if constexpr (N == 1) asm volatile("" ::"s"(b[0]));
  if constexpr (N == 2) asm volatile("" ::"s"(b[0]), "s"(b[1]));
  if constexpr (N == 3) asm volatile("" ::"s"(b[0]), "s"(b[1]), "s"(b[2]));
  if constexpr (N == 4) asm volatile("" ::"s"(b[0]), "s"(b[1]), "s"(b[2]), "s"(b[3]));
}

// The bits every valid lane's value shares, as (prefix, top): prefix holds
// the common bits above the highest bit in which two valid values differ,
// zeros from that bit down; top is that bit (-1 if all agree, i.e. prefix
// is the common value, or if no lane is valid).  a and o are the lane's own
// AND and OR over its valid values (~0 and 0 if none).
__device__ __forceinline__ uint32_t common_prefix(uint32_t a, uint32_t o, int& top) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a &= static_cast<uint32_t>(__shfl_xor(static_cast<int>(a), off, 64));
    o |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(o), off, 64));
  }
  const uint32_t d = a ^ o;
  if (o == 0u && a == ~0u) {  // no valid lane
    top = 31;
    return 0u;
  }
  top = d ? 31 - __builtin_clz(d) : -1;
  return d ? (o & ~((2u << top) - 1u)) : o;
}

// The float whose value key is v (v >= 1 and the key of a number).
__device__ __forceinline__ uint32_t key_bits(uint32_t v) { return (v & 0x80000000u) ? (v ^ 0x80000000u) : ~v; }

// Appends the elements of one lane-column that pass to the survivor list.
__device__ __forceinline__ void compact_one(WaveShared& sh, int& count, bool take, uint32_t bits, uint32_t li) {
  const uint64_t m = __ballot(take);
  if (take) {
    uint32_t slot = lanes_below(m, static_cast<uint32_t>(count));
    slot = slot < CAND ? slot : CAND;
    sh.bits[slot] = bits;
    sh.li[slot] = li;
  }
  count += __popcll(m);
}

__device__ __forceinline__ void compact_key(MergeShared& sh, int& count, bool take, uint64_t key) {
  const uint64_t m = __ballot(take);
  if (take) {
    uint32_t slot = lanes_below(m, static_cast<uint32_t>(count));
    slot = slot < CAND ? slot : CAND;
    sh.key[slot] = key;
  }
  count += __popcll(m);
}

// Ranks the c <= 64*E survivors and writes those of rank < K.  CO: the
// reload of survivors' bits (exact path) reads X at device coherence.
template <int E, bool CO>
__device__ __forceinline__ void rank_and_write(WaveShared& sh, int c, int K, int base, int chunks,
                                               int64_t row, int chunk, const float* __restrict__ xc,
                                               bool reload, uint64_t* __restrict__ ws,
                                               float* __restrict__ out_vals,
                                               int32_t* __restrict__ out_idx, int64_t ld_out) {
  const int lane = threadIdx.x & 63;
  uint32_t b[E], l[E];
  uint64_t k[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int s = lane + 64 * r;
    const bool live = s < c;
    l[r] = live ? sh.li[s] : 0u;
    float xv = 0.f;
    if (live && reload)
      xv = CO ? __hip_atomic_load(xc + l[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : xc[l[r]];
    b[r] = live ? (reload ? __builtin_bit_cast(uint32_t, xv) : sh.bits[s]) : 0u;
    k[r] = live ? ((static_cast<uint64_t>(vs::value_key(b[r])) << 32) |
                   static_cast<uint32_t>(~static_cast<uint32_t>(base + static_cast<int>(l[r]))))
                : 0ull;
    sh.key[s] = k[r];  // empty slots hold 0, which is below every key
  }
  vs::wave_lds_sync();
  int rank[E];
#pragma unroll
  for (int r = 0; r < E; ++r) rank[r] = 0;
  const int cr = (c + 15) & ~15;  // <= 64*E; keys past c are 0
  for (int s = 0; s < cr; s += 16) {
    uint64_t q[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) q[u] = sh.key[s + u];
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int r = 0; r < E; ++r) rank[r] += q[u] > k[r];
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

// Chunk stage: one wavefront per (row, chunk of up to 64 * NPL elements).
//
// Lane l holds NPL values of the chunk (element j of the lane is chunk index
// 256*(j/4) + 4*l + j%4, so every load is a coalesced 1 KB), in GROUPS groups
// per lane.  Steps, each cheap in vector instructions:
//   1. the float maximum of each group (NaN is skipped or, if signalling,
//      makes the maximum NaN: either way the group holds an element at
//      least as large, in key order, as the maximum found);
//   2. v = the K-th largest value key of the group maxima, by a bitwise
//      search on ballot counts.  The K groups at or above v hold K distinct
//      elements of value key >= v, so the top K are among the elements with
//      value key >= v: those above v, and of those equal to v (a tie, also
//      the all-equal row) only the ones with the lowest indices, as many as
//      the elements above v leave to fill.  With t the float whose key is v
//      these are the float comparisons x > t and x == t (NaN passes neither,
//      -0 and +0 compare equal as their keys do; fp32 denormals are kept, so
//      the comparisons are exact);
//   3. the survivors (a few dozen on ordinary rows) are compacted to LDS as
//      (bits, chunk index) pairs;
//   4. each survivor's rank is the number of larger 64-bit keys among them;
//      ranks below K are the output positions.
// If fewer than K group maxima are real numbers, every valid element
// survives.  If more than CAND survive (adversarial rows, where the top
// values crowd into a few lanes), the threshold is made exact: the K-th
// largest value key of all the chunk's elements, by the same bitwise search,
// leaves exactly K survivors after the same compaction.  Either way the
// result is exact: keys are unique.
//
// pre(x, xrow, base, n) runs once the lane's values are loaded: a hook that
// may change values of the chunk in the registers (and in X); CO: a hook
// wrote into X, so the exact path waits for those stores and its reload of
// survivors reads X coherently.
struct NoPre {
  template <int NPL>
  __device__ __forceinline__ void operator()(float (&)[NPL], float*, int, int) const {}
};

template <int NPL, int GROUPS, bool CO, class Pre>
__device__ __forceinline__ void chunk_unit(WaveShared& sh, const float* __restrict__ X, int64_t ldx, int row,
                                           int chunk, int V, int K, int chunks, uint64_t* __restrict__ ws,
                                           float* __restrict__ out_vals, int32_t* __restrict__ out_idx,
                                           int64_t ld_out, const Pre& pre) {
  constexpr int CH = 64 * NPL;
  constexpr int GL = NPL / GROUPS;
  static_assert(NPL % 4 == 0 && GL >= 3, "chunk shape");
  const int lane = threadIdx.x & 63;
  const float* xrow = X + static_cast<int64_t>(row) * ldx;
  const int base = chunk * CH;
  const int n = V - base < CH ? V - base : CH;

  // the lane's NPL values; elements past the row's end read as NaN, which
  // no maximum or threshold comparison selects
  float x[NPL];
  const bool vec = n == CH && ((reinterpret_cast<uintptr_t>(xrow + base) & 15u) == 0);
  if (vec) {
#pragma unroll
    for (int q = 0; q < NPL / 4; ++q) {
      // non-temporal: each value is read once (1-2% faster on batches)
      const f32x4 f = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xrow + base + (q << 8) + (lane << 2)));
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
  pre(x, const_cast<float*>(xrow), base, n);

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
  // one bit per step, unrolled (a single wave runs this search, so its
  // instruction count is its time).  Below bit COARSE_BIT the search goes on
  // only while more than K + COARSE_SLACK maxima are at or above v: the
  // threshold may stay a lower bound of the K-th largest maximum (at least
  // K maxima at or above it), so the survivors still hold the top K, ranked
  // exactly below, plus the few elements just under the K-th maximum.
  uint32_t v = 0;
  int nv = 64 * GROUPS;  // maxima at or above v
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    if (bit < COARSE_BIT && nv <= K + COARSE_SLACK) break;  // uniform
    const uint32_t c = v | (1u << bit);
    uint64_t b[GROUPS];
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) b[g] = __ballot(mk[g] >= c);
    pin_ballots(b);
    int n = 0;
#pragma unroll
    for (int g = 0; g < GROUPS; ++g) n += __popcll(b[g]);
    if (n >= K) {
      v = c;
      nv = n;
    }
  }
  // below -inf's key only NaN patterns (no value key) lie: a cleared
  // threshold there stands for -inf, which the same maxima reach
  if (v != 0u && v < NEG_INF_KEY) v = NEG_INF_KEY;

  // 3: compaction: the elements above t and, of those equal to t, the ones
  // with the lowest chunk indices, until K are taken
  const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
  int count = 0;
  if (v != 0) {
    const float t = __builtin_bit_cast(float, key_bits(v));
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      compact_one(sh, count, x[j] > t, __builtin_bit_cast(uint32_t, x[j]),
                  lane4 | static_cast<uint32_t>(((j >> 2) << 8) | (j & 3)));
    const int need = K - count;  // ties still to take, lowest index first
    if (need > 0) {
      int ties_before = 0;  // in the 256-element blocks already passed
#pragma unroll
      for (int q = 0; q < NPL / 4; ++q) {
        // within block q, chunk index order is lane-major, then j % 4
        uint64_t tb[4];
        int below = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          tb[r] = __ballot(x[4 * q + r] == t);
          below += static_cast<int>(lanes_below(tb[r]));
        }
        int own = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool tie = ((tb[r] >> lane) & 1ull) != 0;
          compact_one(sh, count, tie && ties_before + below + own < need,
                      __builtin_bit_cast(uint32_t, x[4 * q + r]), lane4 | static_cast<uint32_t>((q << 8) | r));
          own += tie;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) ties_before += __popcll(tb[r]);
        if (ties_before >= need) break;  // uniform: no later tie is taken
      }
    }
  } else {  // fewer than K group maxima are numbers: every valid element
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int li = chunk_index(lane, j);
      compact_one(sh, count, li < n, __builtin_bit_cast(uint32_t, x[j]), static_cast<uint32_t>(li));
    }
  }

  const bool exact = count > CAND;
  if (exact) {
    // CO: the hook's stores into X are complete before the survivors' bits
    // are read back from it
    if constexpr (CO) __builtin_amdgcn_s_waitcnt(0);
    // the exact K-th largest value key of the chunk, by the same bitwise
    // search over every element's value key (padding is NaN, value key 0,
    // and ranks after every valid element of that key), then the same
    // compaction: exactly K survivors.  x is turned into value keys in
    // place; the survivors' bits are read again for output.
#pragma unroll
    for (int j = 0; j < NPL; ++j) x[j] = __builtin_bit_cast(float, vs::value_key(__builtin_bit_cast(uint32_t, x[j])));
    uint32_t vt = 0;  // (one bit per step: this rare path keeps its scalar registers few)
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = vt | (1u << bit);
      int c = 0;
#pragma unroll
      for (int j = 0; j < NPL; ++j) c += __popcll(__ballot(__builtin_bit_cast(uint32_t, x[j]) >= cand));
      if (c >= K) vt = cand;
    }
    count = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      compact_one(sh, count, __builtin_bit_cast(uint32_t, x[j]) > vt, __builtin_bit_cast(uint32_t, x[j]),
                  lane4 | static_cast<uint32_t>(((j >> 2) << 8) | (j & 3)));
    const int need = K - count;  // ties still to take, lowest index first
    if (need > 0) {
      int ties_before = 0;  // in the 256-element blocks already passed
#pragma unroll
      for (int q = 0; q < NPL / 4; ++q) {
        // within block q, chunk index order is lane-major, then j % 4
        uint64_t tb[4];
        int below = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          tb[r] = __ballot(__builtin_bit_cast(uint32_t, x[4 * q + r]) == vt);
          below += static_cast<int>(lanes_below(tb[r]));
        }
        int own = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool tie = ((tb[r] >> lane) & 1ull) != 0;
          compact_one(sh, count, tie && ties_before + below + own < need,
                      __builtin_bit_cast(uint32_t, x[4 * q + r]), lane4 | static_cast<uint32_t>((q << 8) | r));
          own += tie;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) ties_before += __popcll(tb[r]);
        if (ties_before >= need) break;  // uniform: no later tie is taken
      }
    }
  }

  // 4: ranks and output
  if (count > CAND) count = CAND;  // not reached: the exact threshold leaves K
  vs::wave_lds_sync();
  const float* xc = xrow + base;
  if (count <= 64)
    rank_and_write<1, CO>(sh, count, K, base, chunks, row, chunk, xc, exact, ws, out_vals, out_idx, ld_out);
  else if (count <= 128)
    rank_and_write<2, CO>(sh, count, K, base, chunks, row, chunk, xc, exact, ws, out_vals, out_idx, ld_out);
  else
    rank_and_write<4, CO>(sh, count, K, base, chunks, row, chunk, xc, exact, ws, out_vals, out_idx, ld_out);
}

// The K-th largest of the wave's keys k[0..N) (0 = empty slot), or 0 if
// fewer than K are non-zero.  A bitwise search, two bits per step, first
// over the value keys (high halves), then, only if more keys than needed
// share the value key found, over the index halves of those ties.  When
// the ties are exactly as many as needed the result is the value key with
// a zero index half: the same keys, exactly K, are at or above it.
//
// COARSE: below bit COARSE_BIT the search over the value keys goes on only
// while more than K + COARSE_SLACK keys are at or above it; if it stops
// there, the result is that value key with a zero index half: a lower bound
// of the K-th largest key with at least K keys at or above it (0 if fewer
// than K keys are non-zero), for callers that rank their survivors exactly.
// Otherwise (every value bit searched: ties, or keys crowded within 2^-7)
// the index halves are searched as without COARSE.
template <int N, bool COARSE = false>
__device__ __forceinline__ uint64_t wave_kth_largest(const uint64_t (&k)[N], int K) {
  uint32_t hi[N], lo[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    hi[i] = static_cast<uint32_t>(k[i] >> 32);
    lo[i] = static_cast<uint32_t>(k[i]);
  }
  // the search starts below the bits all real keys share: the K-th largest
  // shares them too (a candidate that sets a shared bit is either unchanged
  // or above every key, so the choice at each step is the same)
  uint32_t la = ~0u, lo_or = 0u;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (k[i] != 0ull) {
      la &= hi[i];
      lo_or |= hi[i];
    }
  }
  int top;
  uint32_t vh = common_prefix(la, lo_or, top);
  int nv = 0;  // COARSE: non-zero keys at or above vh (at first all, which share its bits)
  if constexpr (COARSE) {
#pragma unroll
    for (int i = 0; i < N; ++i) nv += __popcll(__ballot(k[i] != 0ull));
  }
  bool stopped = false;  // COARSE: the search ended above bit 0
  // one bit per step, unrolled, from the highest bit in which keys differ
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    if (bit > top) continue;  // uniform: a bit every key shares
    if (COARSE && bit < COARSE_BIT && nv <= K + COARSE_SLACK) {  // uniform
      stopped = true;
      break;
    }
    const uint32_t c = vh | (1u << bit);
    uint64_t b[N];
#pragma unroll
    for (int i = 0; i < N; ++i) b[i] = __ballot(hi[i] >= c);
    pin_ballots(b);
    int n = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) n += __popcll(b[i]);
    if (n >= K) {
      vh = c;
      nv = n;
    }
  }
  if (COARSE && stopped) return nv >= K ? static_cast<uint64_t>(vh) << 32 : 0ull;
  // index halves of the ties, 0 for the other keys (an index half is the
  // complement of an index below 2^31, so a real one is never 0)
  int above = 0, ties = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bool real = k[i] != 0ull;
    const bool tie = real && hi[i] == vh;
    lo[i] = tie ? lo[i] : 0u;
    above += __popcll(__ballot(real && hi[i] > vh));
    ties += __popcll(__ballot(tie));
  }
  const int need = K - above;
  if (need > ties) return 0ull;  // fewer than K keys
  const uint64_t base = static_cast<uint64_t>(vh) << 32;
  if (need == ties) return base;
  la = ~0u;
  lo_or = 0u;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (lo[i] != 0u) {
      la &= lo[i];
      lo_or |= lo[i];
    }
  }
  uint32_t vl = common_prefix(la, lo_or, top);
  for (int bit = (top | 1) - 1; bit >= 0; bit -= 2) {
    const uint32_t c1 = vl | (1u << bit), c2 = vl | (2u << bit), c3 = vl | (3u << bit);
    int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      uint32_t l = lo[i];
      asm volatile("" : "+v"(l));
      const uint64_t b1 = __ballot(l >= c1), b2 = __ballot(l >= c2), b3 = __ballot(l >= c3);
      pin3(b1, b2, b3);
      n1 += __popcll(b1);
      n2 += __popcll(b2);
      n3 += __popcll(b3);
    }
    vl = n3 >= need ? c3 : (n2 >= need ? c2 : (n1 >= need ? c1 : vl));
  }
  return base | vl;
}

// The input bits of the element a key stands for, when the key fixes them
// (every value but NaN, whose payload, and zero, whose sign, it drops).
__device__ __forceinline__ bool bits_of_key(uint64_t key, uint32_t& bits) {
  const uint32_t vk = static_cast<uint32_t>(key >> 32);
  if (vk == 0u || vk == 0x80000000u) return false;
  bits = (vk & 0x80000000u) ? (vk & 0x7fffffffu) : ~vk;
  return true;
}

// Ranks the c <= 64*E merge survivors and writes those of rank < K.
template <int E>
__device__ __forceinline__ void merge_rank_write(MergeShared& sh, int c, int K, int V, const float* __restrict__ xrow,
                                                 float* ovals, int32_t* oidx) {
  const int lane = threadIdx.x & 63;
  uint64_t k[E];
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int s = lane + 64 * r;
    k[r] = s < c ? sh.key[s] : 0ull;
  }
  vs::wave_lds_sync();  // every lane has its key before the tail is cleared
#pragma unroll
  for (int r = 0; r < E; ++r) {
    const int s = lane + 64 * r;
    if (s >= c) sh.key[s] = 0ull;  // below every key
  }
  vs::wave_lds_sync();
  int rank[E];
#pragma unroll
  for (int r = 0; r < E; ++r) rank[r] = 0;
  const int cr = (c + 15) & ~15;  // <= 64*E; keys past c are 0
  for (int s = 0; s < cr; s += 16) {
    uint64_t q[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) q[u] = sh.key[s + u];
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int r = 0; r < E; ++r) rank[r] += q[u] > k[r];
  }
#pragma unroll
  for (int r = 0; r < E; ++r) {
    if (lane + 64 * r < c && rank[r] < K) {
      const uint32_t idx = vs::key_index(k[r]);
      uint32_t bits;
      if (!bits_of_key(k[r], bits)) bits = __builtin_bit_cast(uint32_t, xrow[idx < static_cast<uint32_t>(V) ? idx : 0u]);
      oidx[rank[r]] = static_cast<int32_t>(idx);
      ovals[rank[r]] = __builtin_bit_cast(float, bits);  // the input's bits
    }
  }
  if (lane >= c && lane < K) {  // fewer than K elements: empty entries
    oidx[lane] = -1;
    ovals[lane] = __builtin_nanf("");
  }
}

// Merge of a row whose chunk maxima are the threshold's entries and fit three
// to a lane (K <= chunks <= 192, K even), lane-major: lane l holds the first
// WIDE_READ entries of chunks l, l + 64 and l + 128.  With v the K-th
// largest chunk maximum (as in merge_row, step 1), each chunk's survivors
// (keys >= v) are a prefix of its sorted list, so their positions in the
// survivor list follow from one prefix sum of the per-lane counts over the
// lanes (five ballots of the counts' bits), with no compaction rounds.
// A chunk whose WIDE_READ entries all survive ("full") may hold more
// survivors further down its list.  Only chunks with a maximum >= v can be
// full, at most K of them, so when their unread entries fit WIDE_EXTRA loads
// per lane (K (K - WIDE_READ) <= 64 WIDE_EXTRA: K <= 16) they are read in
// one more round and their survivors appended.  This is what rows whose top
// K crowds into the first chunks need (equal values, many -inf: ties go to
// the lowest indices).  Returns false, having written only LDS, when full
// chunks hold more than that or more than CAND keys survive; merge_row then
// takes its general path.
constexpr int WIDE_SLOTS = 3;
constexpr int WIDE_READ = 8;
constexpr int WIDE_EXTRA = 2;
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bool merge_row_wide(MergeShared& sh, const uint64_t* __restrict__ src, int chunks, int K,
                                               int& count) {
  const int lane = threadIdx.x & 63;
  uint64_t e[WIDE_SLOTS][WIDE_READ];
#pragma unroll
  for (int s = 0; s < WIDE_SLOTS; ++s) {
    const int c = lane + 64 * s;
#pragma unroll
    for (int j = 0; j < WIDE_READ; j += 2) {
      u64x2 pr = {0ull, 0ull};
      if (c < chunks) pr = *reinterpret_cast<const u64x2*>(src + c * K + j);  // K even: 16-byte aligned
      e[s][j] = pr.x;
      e[s][j + 1] = pr.y;
    }
  }
  uint64_t m[WIDE_SLOTS];
#pragma unroll
  for (int s = 0; s < WIDE_SLOTS; ++s) m[s] = e[s][0];  // 0 for chunks past the row's
  const uint64_t v = wave_kth_largest<WIDE_SLOTS, true>(m, K);
  int n[WIDE_SLOTS];
  int total = 0;
  bool full = false;
#pragma unroll
  for (int s = 0; s < WIDE_SLOTS; ++s) {
    n[s] = 0;
#pragma unroll
    for (int j = 0; j < WIDE_READ; ++j) n[s] += e[s][j] != 0ull && e[s][j] >= v;
    total += n[s];
    full = full || n[s] == WIDE_READ;
  }
  const bool any_full = K > WIDE_READ && __ballot(full) != 0ull;  // uniform
  if (any_full && K * (K - WIDE_READ) > 64 * WIDE_EXTRA) return false;
  // exclusive prefix of total over the lanes (total <= 24: five bits)
  int pos = 0;
  count = 0;
#pragma unroll
  for (int b = 0; b < 5; ++b) {
    const uint64_t bb = __ballot((total >> b) & 1);
    pos += static_cast<int>(lanes_below(bb)) << b;
    count += __popcll(bb) << b;
  }
  if (count > CAND) return false;  // uniform
#pragma unroll
  for (int s = 0; s < WIDE_SLOTS; ++s)
#pragma unroll
    for (int j = 0; j < WIDE_READ; ++j)
      if (j < n[s]) sh.key[pos++] = e[s][j];
  if (any_full) {
    // the full chunks, in (slot, lane) order, listed in LDS (at most K)
    int nf = 0;
#pragma unroll
    for (int s = 0; s < WIDE_SLOTS; ++s) {
      const uint64_t bf = __ballot(n[s] == WIDE_READ);
      if (n[s] == WIDE_READ) sh.cont[nf + static_cast<int>(lanes_below(bf))] = static_cast<uint32_t>(lane + 64 * s);
      nf += __popcll(bf);
    }
    vs::wave_lds_sync();
    // their entries WIDE_READ .. K - 1: entry q of the round is entry
    // WIDE_READ + q % U of full chunk q / U
    const int U = K - WIDE_READ;
    if (nf * U > 64 * WIDE_EXTRA) return false;  // uniform; not reached while nf <= K
    uint64_t x[WIDE_EXTRA];
    int t = 0;
#pragma unroll
    for (int i = 0; i < WIDE_EXTRA; ++i) {
      const int q = lane + 64 * i;
      x[i] = 0ull;
      if (q < nf * U) x[i] = src[static_cast<int64_t>(sh.cont[q / U]) * K + WIDE_READ + q % U];
      t += x[i] != 0ull && x[i] >= v;
    }
    // appended after the first survivors: exclusive prefix of t (<= 2: two bits)
    int pos2 = count, extra = 0;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const uint64_t bb = __ballot((t >> b) & 1);
      pos2 += static_cast<int>(lanes_below(bb)) << b;
      extra += __popcll(bb) << b;
    }
    if (count + extra > CAND) return false;  // uniform
#pragma unroll
    for (int i = 0; i < WIDE_EXTRA; ++i)
      if (x[i] != 0ull && x[i] >= v) sh.key[pos2++] = x[i];
    count += extra;
  }
  return true;
}

// Merge stage: one wavefront per row over the chunks' candidate lists (K
// keys per chunk, sorted descending, zero-padded).
//   1. v = the K-th largest key among the first jp entries of every chunk
//      (jp = 1 when there are at least K chunks), by a bitwise search on
//      ballot counts: those K keys are candidates, so every top-K key is
//      >= v;
//   2. the survivors, keys >= v, are a prefix of each chunk's list.  The
//      first j2 entries of every chunk are read in one round
//      (chunks * j2 <= 64 * MERGE_LOADS); the chunks whose j2 entries all
//      survive are read on to the end of their lists;
//   3. ranks among the survivors, as in the chunk stage.
// More than CAND survivors (ties resolved by index crowd the top K into the
// first chunks, as in the all-equal row with K = 64) take a second,
// narrower round whose survivors are bounded by CAND.  Rows of K to 192
// chunks first try merge_row_wide, steps 1-2 in fewer instructions.
// ovals, oidx: the row's K outputs (global or LDS).
__device__ __forceinline__ void merge_row(MergeShared& sh, const float* __restrict__ X, int64_t ldx, int row,
                                          int V, int K, int chunks, int lg_jp, int lg_j2,
                                          const uint64_t* __restrict__ ws, float* ovals, int32_t* oidx) {
  const int lane = threadIdx.x & 63;
  const int n = chunks * K;
  const uint64_t* src = ws + static_cast<int64_t>(row) * n;
  const int jp = 1 << lg_jp, j2 = 1 << lg_j2;
  int count = 0;
  const bool wide = lg_jp == 0 && chunks <= 64 * WIDE_SLOTS && (K & 1) == 0 && K >= WIDE_READ &&
                    merge_row_wide(sh, src, chunks, K, count);
  if (!wide) {
    // both reads in one round: the threshold's entries (chunks * jp <= 256)
    // and the first j2 entries of every chunk
    uint64_t m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = lane + 64 * i;
      const int c = t >> lg_jp, j = t & (jp - 1);
      m[i] = (c < chunks && j < K) ? src[c * K + j] : 0ull;
    }
    uint64_t e[MERGE_LOADS];
    const int n2 = chunks << lg_j2;
#pragma unroll
    for (int i = 0; i < MERGE_LOADS; ++i) {
      e[i] = 0ull;
      if (64 * i < n2) {  // uniform
        const int s = lane + 64 * i;
        const int c = s >> lg_j2, j = s & (j2 - 1);
        if (c < chunks && j < K) e[i] = src[c * K + j];
      }
    }

    // 1: the K-th largest key of the threshold's entries (0 if fewer than K)
    const uint64_t v = wave_kth_largest<4>(m, K);

    // 2: survivors of the first round, and the chunks to read on
    count = 0;
    int n_cont = 0;
#pragma unroll
    for (int i = 0; i < MERGE_LOADS; ++i) {
      if (64 * i < n2) {
        const bool live = e[i] != 0ull && e[i] >= v;
        compact_key(sh, count, live, e[i]);
        if (j2 < K) {
          const int s = lane + 64 * i;
          const bool more = live && (s & (j2 - 1)) == j2 - 1;  // its chunk's last entry read
          const uint64_t mm = __ballot(more);
          if (more) sh.cont[lanes_below(mm, static_cast<uint32_t>(n_cont))] = static_cast<uint32_t>(s >> lg_j2);
          n_cont += __popcll(mm);
        }
      }
    }
    vs::wave_lds_sync();
    if (n_cont > 0 && count <= CAND) {
      // entries j2 .. K-1 of those chunks, P (a power of two >= K - j2) lanes per chunk
      const int tail = K - j2;
      const int lg_p = tail <= 1 ? 0 : 32 - __builtin_clz(static_cast<unsigned>(tail - 1));
      const int total = n_cont << lg_p;
      for (int s0 = 0; s0 < total && count <= CAND; s0 += 64 * 8) {
        uint64_t f[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int s = s0 + 64 * u + lane;
          const int j = j2 + (s & ((1 << lg_p) - 1));
          f[u] = 0ull;
          if (s < total && j < K) f[u] = src[static_cast<int>(sh.cont[s >> lg_p]) * K + j];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) compact_key(sh, count, f[u] != 0ull && f[u] >= v, f[u]);
      }
    }

    if (count > CAND) {
      // Second round.  Only the chunks whose first entry is >= v can hold a
      // top-K key: exactly K of them when jp = 1, else at most chunks < K.
      // Their first jb entries (nrel * jb <= 64 * MERGE_LOADS, so jb >= 16
      // when jb < K) give the exact K-th largest key v2 of that set; exactly
      // K read entries are >= v2, so at most K / jb chunks have all jb read
      // entries >= v2, and only those are read on.  That bounds the
      // survivors by K * K / jb <= CAND.
      vs::wave_lds_sync();  // the first round's survivors are dropped
      int nrel = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = lane + 64 * i;
        const bool rel = m[i] != 0ull && m[i] >= v && (t & (jp - 1)) == 0;
        const uint64_t mm = __ballot(rel);
        if (rel) sh.cont[lanes_below(mm, static_cast<uint32_t>(nrel))] = static_cast<uint32_t>(t >> lg_jp);
        nrel += __popcll(mm);
      }
      vs::wave_lds_sync();
      int lg_jb = 31 - __builtin_clz(static_cast<unsigned>((64 * MERGE_LOADS) / (nrel > 0 ? nrel : 1)));
      const int lg_k = K <= 1 ? 0 : 32 - __builtin_clz(static_cast<unsigned>(K - 1));
      lg_jb = lg_jb < lg_k ? lg_jb : lg_k;
      const int jb = 1 << lg_jb;
      const int nb = nrel << lg_jb;
#pragma unroll
      for (int i = 0; i < MERGE_LOADS; ++i) {
        e[i] = 0ull;
        if (64 * i < nb) {  // uniform
          const int s = lane + 64 * i;
          const int r = s >> lg_jb, j = s & (jb - 1);
          if (r < nrel && j < K) e[i] = src[static_cast<int>(sh.cont[r]) * K + j];
        }
      }
      // (one bit per step: this rare path keeps its scalar registers few)
      uint64_t v2 = 0;
      for (int bit = 63; bit >= 0; --bit) {
        const uint64_t cand = v2 | (1ull << bit);
        int c = 0;
#pragma unroll
        for (int i = 0; i < MERGE_LOADS; ++i)
          if (64 * i < nb) c += __popcll(__ballot(e[i] >= cand));
        if (c >= K) v2 = cand;
      }
      count = 0;
      int nlong = 0;
#pragma unroll
      for (int i = 0; i < MERGE_LOADS; ++i) {
        if (64 * i < nb) {
          const int s = lane + 64 * i;
          const bool live = e[i] != 0ull && e[i] >= v2;
          compact_key(sh, count, live, e[i]);
          if (jb < K) {
            const bool more = live && (s & (jb - 1)) == jb - 1;
            const uint64_t mm = __ballot(more);
            // after the relevant list (<= 64 entries)
            if (more) sh.cont[64 + lanes_below(mm, static_cast<uint32_t>(nlong))] = sh.cont[s >> lg_jb];
            nlong += __popcll(mm);
          }
        }
      }
      vs::wave_lds_sync();
      // entries jb .. K-1 of at most K / jb <= 4 chunks, 64 lanes per chunk
      for (int u0 = 0; u0 < nlong; u0 += 4) {
        uint64_t f[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = jb + lane;
          f[u] = 0ull;
          if (u0 + u < nlong && j < K) f[u] = src[static_cast<int>(sh.cont[64 + u0 + u]) * K + j];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) compact_key(sh, count, f[u] != 0ull && f[u] >= v2, f[u]);
      }
    }
  }  // general path

  if (count > CAND) count = CAND;  // not reached: the rounds above bound the survivors
  vs::wave_lds_sync();
  if (count > 128) {
    // ranking costs grow with the square of the survivors: cut them to
    // exactly K first, at the exact K-th largest of them
    uint64_t r4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = lane + 64 * r;
      r4[r] = t < count ? sh.key[t] : 0ull;
    }
    const uint64_t v3 = wave_kth_largest<4>(r4, K);
    vs::wave_lds_sync();  // every lane has its keys before the list is rewritten
    count = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) compact_key(sh, count, r4[r] != 0ull && r4[r] >= v3, r4[r]);
    vs::wave_lds_sync();
  }
  const float* xrow = X + static_cast<int64_t>(row) * ldx;
  if (count <= 64)
    merge_rank_write<1>(sh, count, K, V, xrow, ovals, oidx);
  else if (count <= 128)
    merge_rank_write<2>(sh, count, K, V, xrow, ovals, oidx);
  else
    merge_rank_write<4>(sh, count, K, V, xrow, ovals, oidx);
}

// Which chunking a call takes; the workspace size follows from it.
struct Plan {
  bool small;  // 1024-element chunks
  int chunks;
};

inline Plan plan_for(int rows, int V) {
  const int large = (V + LARGE_CHUNK - 1) / LARGE_CHUNK;
  const bool small = V <= SMALL_CHUNK ||
                     (large > 1 && static_cast<int64_t>(rows) * large < SMALL_BATCH_UNITS);
  return {small, small ? (V + SMALL_CHUNK - 1) / SMALL_CHUNK : large};
}

inline int log2_floor(int x) { return 31 - __builtin_clz(static_cast<unsigned>(x)); }
inline int log2_ceil(int x) { return x <= 1 ? 0 : 32 - __builtin_clz(static_cast<unsigned>(x - 1)); }

// The merge's read lengths: threshold entries jp per chunk with chunks * jp
// >= K; first read j2 per chunk, the most that fit one round, and no more
// than the lists hold (as log2).
inline void merge_reads(int chunks, int K, int& lg_jp, int& lg_j2) {
  lg_jp = chunks >= K ? 0 : log2_ceil((K + chunks - 1) / chunks);
  lg_j2 = log2_floor((64 * MERGE_LOADS) / chunks);
  if (lg_j2 > log2_ceil(K)) lg_j2 = log2_ceil(K);
}

}  // namespace
