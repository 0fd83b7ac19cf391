// tree_attention_rows: attention of a token tree's verify rows over the
// context KV cache and the tree's KV scratch slots, under the tree mask;
// tree_commit_kv: the accepted branch's scratch slots written into the cache.
//
// "One RDNA4 verify pass has slack for about two dozen speculative tokens":
// "Spend the budget on a tree, not a longer guess" (one pass verifies several
// branches sharing a prefix; the attention mask is tree-shaped, each branch
// attending only to its ancestors), "Where the tree earns its keep" (the
// candidates' keys and values go to scratch slots and only the accepted
// branch is kept), "What I am building toward" (the mask folded into the
// decode kernel).
//
// Rows and slots: row 0 is the root (scratch slot 0), row 1 + j is node j
// (slot 1 + j); row r sees every context position and the slots of its
// ancestors and itself (the path from node j follows parent[] up to the
// root, stopping at a parent outside [-1, child)).
//
// Design (MI355X): split-KV decoding.  A workgroup takes one KV head and one
// split of the keys: NB sub-blocks of 64 context positions, or the scratch
// slots (<= 64) under the tree mask.  All G * R query vectors of the KV
// head's G query heads are processed together, so every key and value is
// read once per workgroup: the M = G * R queries are the rows of
// v_mfma_f32_16x16x32_bf16 tiles, split among the four waves.
//  * scores: queries (fp32, split exactly into three bf16 planes hi + mid +
//    lo) times keys (bf16, the B operand straight from HBM); exact products,
//    fp32 accumulation over the 128 head dimensions in a fixed order;
//  * softmax: online over the sub-blocks in fp32 (running maximum m, sum l,
//    rescale by exp(m_old - m_new)); each row's maximum and sum over a
//    sub-block reduce across the 16 lanes of a row group in a fixed order;
//  * values: the probabilities, split exactly into three bf16 planes in
//    registers (the A operand), times V staged transposed in LDS (the B
//    operand, its keys in the order the probabilities sit in the lanes);
//  * each split writes its (m, l, unnormalised output) to a workspace; a
//    second kernel merges the splits in split order: out = sum_s o_s
//    e^(m_s - M) / sum_s l_s e^(m_s - M), M = max_s m_s.

#include "vs_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int HD = 128;       // head dimension
constexpr int BKEYS = 64;     // keys per sub-block
constexpr int WAVES = 8;
constexpr int KSTEPS = HD / 32;     // MFMA k-steps over the head dimension
constexpr int NT_S = BKEYS / 16;    // key tiles of a sub-block
constexpr int NT_O = HD / 16;       // dimension tiles of the output
constexpr int VSTR = BKEYS + 8;     // LDS row stride (bf16) of V transposed
constexpr int MAX_ROWS = 64;        // tree rows (root + up to 63 nodes)
constexpr int MAX_QUERIES = 256;    // G * R per KV head

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bitsf(uint32_t b) { return __builtin_bit_cast(float, b); }

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// x == hi + mid + lo exactly for eight fp32 values (truncation leaves at most
// 16, then 8 significant bits, each exactly a bf16)
__device__ __forceinline__ void split3(const float (&x)[8], u32x4& hi, u32x4& mid, u32x4& lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t h0 = fbits(x[2 * p]) & 0xffff0000u, h1 = fbits(x[2 * p + 1]) & 0xffff0000u;
    const float r0 = x[2 * p] - bitsf(h0), r1 = x[2 * p + 1] - bitsf(h1);
    const uint32_t m0 = fbits(r0) & 0xffff0000u, m1 = fbits(r1) & 0xffff0000u;
    const float s0 = r0 - bitsf(m0), s1 = r1 - bitsf(m1);
    hi[p] = (h0 >> 16) | h1;
    mid[p] = (m0 >> 16) | m1;
    lo[p] = (fbits(s0) >> 16) | (fbits(s1) & 0xffff0000u);
  }
}

// three bf16 pieces of one fp32 value, as 16-bit patterns
__device__ __forceinline__ void split3_one(float x, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
  const uint32_t h = fbits(x) & 0xffff0000u;
  const float r = x - bitsf(h);
  const uint32_t m = fbits(r) & 0xffff0000u;
  const float s = r - bitsf(m);
  hi = static_cast<uint16_t>(h >> 16);
  mid = static_cast<uint16_t>(m >> 16);
  lo = static_cast<uint16_t>(fbits(s) >> 16);
}

// e^x through the hardware base-2 exponential: x * log2(e) rounds once
// (relative error |x| * 2^-24, |x| < ~100 here) and v_exp_f32 adds about
// one ulp; far inside the tolerance the attention is held to
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Slot of key `key` of a sub-block in the LDS copy of V^T.  Within each
// 32-key chunk the keys sit in the order in which a lane holds them after the
// score product (lane group gg has keys 4 gg + e of the chunk's first 16-key
// tile and 16 + 4 gg + e of its second), so that the probabilities serve as
// the A operand of the value product straight from registers: key
// 16 h + 4 gg + e of the chunk goes to slot 8 gg + 4 h + e.
__device__ __forceinline__ int vslot(int key) {
  const int c = key & 31;
  return (key & ~31) + 8 * ((c & 15) >> 2) + 4 * (c >> 4) + (c & 3);
}

// The scratch slots row `row` attends to, as a bit mask (bit s = slot s).
__device__ __forceinline__ uint64_t ancestor_mask(const int32_t* parent, int row) {
  uint64_t m = 1ull;  // the root's slot
  if (row > 0) {
    int child = row - 1;
    m |= 1ull << (child + 1);
    int q = parent[child];
    while (q > -1 && q < child) {  // indices strictly decrease: at most row steps
      m |= 1ull << (q + 1);
      child = q;
      q = parent[q];
    }
  }
  return m;
}

struct Args {
  const float* q;          // [R][Hq][HD]
  const uint16_t* kc;      // [Hkv][cache_len][HD]
  const uint16_t* vc;
  int64_t cache_len;
  int ctx_len;
  const uint16_t* ks;      // [Hkv][scr_len][HD]
  const uint16_t* vs;
  int scr_len;
  const int32_t* parent;   // [R - 1]
  int R, Hq, Hkv, G;
  float scale;
  int NB;                  // context sub-blocks per split
  int ctx_splits;          // splits over the context; split ctx_splits is the scratch slots
  float* part_o;           // [splits][Hkv][M][HD]
  float* part_ml;          // [splits][Hkv][M][2]
};

// Workgroup (g, split, z): KV head g, one split of its keys, query tiles
// WAVES * MTW * z ..; MTW: 16-query tiles per wave.  QREG:
// the queries' bf16 planes stay in registers for the whole split (else they
// are reloaded and split for every sub-block).
//
// Scores are taken transposed, S^T = K Q^T (A = keys, B = query planes), so
// that lane (g, c) holds query c and keys 16 t + 4 g + e: a query's maximum
// and sum are 16 register values and two shuffles across the lane groups.
// Outputs are O = P V (A = the probability planes, straight from the
// registers that computed them; B = V from LDS, its keys permuted to match,
// see vslot); lane (g, c) then holds queries 4 g + e and dimension c of each
// 16-dimension tile, and takes the rescale factors of its four queries from
// the lanes that own them.
template <int MTW, bool QREG>
__global__ void __launch_bounds__(64 * WAVES)
tree_attention_split_kernel(Args a) {
  constexpr int KSTR = HD + 8;  // LDS row stride (bf16) of the key block
  __shared__ __align__(16) uint16_t vt[HD * VSTR];                 // values of the sub-block, [dim][slot]
  __shared__ __align__(16) uint16_t kt[BKEYS * KSTR];              // keys of the sub-block, [key][dim]
  __shared__ int32_t par[MAX_ROWS];
  __shared__ uint64_t anc_row[MAX_ROWS];
  const int lane = threadIdx.x & 63;
  const int w = vs::wave_index();
  const int g = blockIdx.x;                 // KV head
  const int split = blockIdx.y;
  const bool scratch = split == a.ctx_splits;
  const int M = a.G * a.R;
  const int col = lane & 15, grp = lane >> 4;
  const int mt0 = blockIdx.z * WAVES * MTW;  // this workgroup's first query tile

  // the tree mask (scratch split only): parents to LDS, one row per thread
  if (scratch) {  // uniform over the workgroup
    for (int t = threadIdx.x; t < a.R - 1; t += 64 * WAVES) par[t] = a.parent[t];
    __syncthreads();
    for (int r = threadIdx.x; r < a.R; r += 64 * WAVES) anc_row[r] = ancestor_mask(par, r);
    __syncthreads();
  }
  // this wave's query tiles: mt = mt0 + w + WAVES * i; lane (g, c) owns
  // query 16 mt + c of each; padding queries past M see slot 0 only and are
  // dropped
  uint64_t anc[MTW];
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
    const int m = (mt0 + w + WAVES * i) * 16 + col;
    anc[i] = (scratch && m < M) ? anc_row[m % a.R] : 1ull;
  }

  // queries as B operands (query c of the tile, dimensions 32 ks + 8 g ..),
  // split into bf16 planes
  auto q_planes = [&](int i, int ks, u32x4& hi, u32x4& mid, u32x4& lo) {
    const int m = (mt0 + w + WAVES * i) * 16 + col;
    float x[8];
    if (m < M) {
      const int r = m % a.R, hq = g * a.G + m / a.R;
      const float* src = a.q + (static_cast<int64_t>(r) * a.Hq + hq) * HD + ks * 32 + grp * 8;
      const float4 x0 = *reinterpret_cast<const float4*>(src);
      const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
      x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
      x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.f;
    }
    split3(x, hi, mid, lo);
  };

  f32x4 o[MTW][NT_O];  // O tiles: lane (g, c), element e = query 4 g + e, dimension 16 t + c
  float rm[MTW], rl[MTW];
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
#pragma unroll
    for (int t = 0; t < NT_O; ++t) o[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    rm[i] = -__builtin_inff();
    rl[i] = 0.f;
  }

  const uint16_t* kbase = scratch ? a.ks + static_cast<int64_t>(g) * a.scr_len * HD
                                  : a.kc + static_cast<int64_t>(g) * a.cache_len * HD;
  const uint16_t* vbase = scratch ? a.vs + static_cast<int64_t>(g) * a.scr_len * HD
                                  : a.vc + static_cast<int64_t>(g) * a.cache_len * HD;
  const int nkeys = scratch ? a.R : a.ctx_len;
  const int first = scratch ? 0 : split * a.NB * BKEYS;
  int nsub = scratch ? 1 : (nkeys - first + BKEYS - 1) / BKEYS;  // sub-blocks of this split
  if (nsub > (scratch ? 1 : a.NB)) nsub = scratch ? 1 : a.NB;

  // this thread's share of a sub-block's keys and values: 16-byte pieces
  // t + 64 WAVES j, piece p = (key p % 64, dimensions 8 (p / 64) ..); keys
  // past the end are zero (their probabilities are zero, and 0 * garbage
  // could be NaN)
  constexpr int PIECES = BKEYS * HD / 8 / (64 * WAVES);
  u32x4 kr[PIECES], vr[PIECES];
  auto load_kv = [&](int p0) {
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
      const int piece = threadIdx.x + 64 * WAVES * j;
      const int key = piece & (BKEYS - 1), d0 = (piece / BKEYS) * 8;
      const bool ok = p0 + key < nkeys;
      const int64_t off = static_cast<int64_t>(p0 + key) * HD + d0;
      kr[j] = ok ? *reinterpret_cast<const u32x4*>(kbase + off) : u32x4{0u, 0u, 0u, 0u};
      vr[j] = ok ? *reinterpret_cast<const u32x4*>(vbase + off) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_kv = [&]() {
#pragma unroll
    for (int j = 0; j < PIECES; ++j) {
      const int piece = threadIdx.x + 64 * WAVES * j;
      const int key = piece & (BKEYS - 1), d0 = (piece / BKEYS) * 8;
      *reinterpret_cast<u32x4*>(&kt[key * KSTR + d0]) = kr[j];
      const int slot = vslot(key);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        vt[(d0 + 2 * jj) * VSTR + slot] = static_cast<uint16_t>(vr[j][jj] & 0xffffu);
        vt[(d0 + 2 * jj + 1) * VSTR + slot] = static_cast<uint16_t>(vr[j][jj] >> 16);
      }
    }
  };

  // the first sub-block's keys and values are in flight while the queries
  // are loaded and split
  if (nsub > 0) load_kv(first);
  u32x4 qp[QREG ? MTW : 1][KSTEPS][3];
  if constexpr (QREG) {
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) q_planes(i, ks, qp[i][ks][0], qp[i][ks][1], qp[i][ks][2]);
  }
  for (int sb = 0; sb < nsub; ++sb) {  // uniform over the workgroup
    const int p0 = first + sb * BKEYS;
    __syncthreads();  // the previous sub-block's kt, vt and planes have been read
    store_kv();
    __syncthreads();
    if (sb + 1 < nsub) load_kv(p0 + BKEYS);  // the next sub-block, in flight meanwhile

    // S^T tiles: A = keys 16 t .. (key c of the tile, dimensions 32 ks + 8 g ..)
    f32x4 s[MTW][NT_S];
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int t = 0; t < NT_S; ++t) s[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 ka[NT_S];
#pragma unroll
      for (int t = 0; t < NT_S; ++t)
        ka[t] = *reinterpret_cast<const u32x4*>(&kt[(t * 16 + col) * KSTR + ks * 32 + grp * 8]);
#pragma unroll
      for (int i = 0; i < MTW; ++i) {
        u32x4 hi, mid, lo;
        if constexpr (QREG) {
          hi = qp[i][ks][0];
          mid = qp[i][ks][1];
          lo = qp[i][ks][2];
        } else {
          q_planes(i, ks, hi, mid, lo);
        }
#pragma unroll
        for (int t = 0; t < NT_S; ++t) {
          s[i][t] = mfma(ka[t], hi, s[i][t]);
          s[i][t] = mfma(ka[t], mid, s[i][t]);
          s[i][t] = mfma(ka[t], lo, s[i][t]);
        }
      }
    }

    // online softmax over the sub-block for the lane's query of each tile;
    // the probabilities are split into the A operands of the value product
    // (chunk kk: keys of tiles 2 kk and 2 kk + 1, in vslot order)
    const bool all_keys = !scratch && p0 + BKEYS <= nkeys;
    u32x4 pa[MTW][BKEYS / 32][3];
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      float bm = -__builtin_inff();
#pragma unroll
      for (int t = 0; t < NT_S; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = t * 16 + 4 * grp + e;  // within the sub-block
          const bool ok = all_keys || (scratch ? (key < a.R && ((anc[i] >> key) & 1ull)) : (p0 + key < nkeys));
          s[i][t][e] = ok ? s[i][t][e] * a.scale : -__builtin_inff();
          bm = fmaxf(bm, s[i][t][e]);
        }
      bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));  // every query sees a key of every sub-block
      const float mn = fmaxf(rm[i], bm);
      const float alpha = fast_exp(rm[i] - mn);  // 0 on the first sub-block
      rm[i] = mn;
      float ps = 0.f;
#pragma unroll
      for (int kk = 0; kk < BKEYS / 32; ++kk) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pv[j] = fast_exp(s[i][2 * kk + j / 4][j % 4] - mn);  // 0 for masked keys
          ps += pv[j];
        }
        split3(pv, pa[i][kk][0], pa[i][kk][1], pa[i][kk][2]);
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      rl[i] = rl[i] * alpha + ps;
      // the rescale factors of this lane's output queries 4 g + e
      float ae[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ae[e] = __shfl(alpha, 4 * grp + e, 64);
#pragma unroll
      for (int t = 0; t < NT_O; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[i][t][e] *= ae[e];
    }

    // O += P V: A = the probability planes (query c, slots 32 kk + 8 g ..),
    // B = V (slots 32 kk + 8 g .., dimension c of the tile)
#pragma unroll
    for (int kk = 0; kk < BKEYS / 32; ++kk) {
      u32x4 vb[NT_O];
#pragma unroll
      for (int t = 0; t < NT_O; ++t)
        vb[t] = *reinterpret_cast<const u32x4*>(&vt[(t * 16 + col) * VSTR + kk * 32 + grp * 8]);
#pragma unroll
      for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int t = 0; t < NT_O; ++t) {
          o[i][t] = mfma(pa[i][kk][0], vb[t], o[i][t]);
          o[i][t] = mfma(pa[i][kk][1], vb[t], o[i][t]);
          o[i][t] = mfma(pa[i][kk][2], vb[t], o[i][t]);
        }
    }
  }

  // partial results of this split: real queries only
  const int64_t base = (static_cast<int64_t>(split) * a.Hkv + g) * M;
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
    const int mb = (mt0 + w + WAVES * i) * 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = mb + 4 * grp + e;
      if (m >= M) continue;
      float* dst = a.part_o + (base + m) * HD + col;
#pragma unroll
      for (int t = 0; t < NT_O; ++t) dst[t * 16] = o[i][t][e];
    }
    const int m = mb + col;
    if (m < M && grp == 0) {
      a.part_ml[(base + m) * 2] = rm[i];
      a.part_ml[(base + m) * 2 + 1] = rl[i];
    }
  }
}

// out[r][hq][d] from the splits' partial results, merged in split order.
// One workgroup per query vector, one thread per dimension.  The first
// PRE splits' partial outputs are loaded together with the statistics (one
// memory round for both); the splits' weights e^(m_s - M) are kept in LDS;
// each thread then adds its dimension over the splits in split order,
// loading any further partial outputs 16 splits at a time.
constexpr int MAX_SPLITS = 260;  // plan_for keeps the context splits of a KV head <= 256
constexpr int PRE = 32;

__global__ void __launch_bounds__(HD)
tree_attention_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                              int splits, int Hkv, int G, int R, int Hq, float* __restrict__ out) {
  __shared__ float f[MAX_SPLITS];   // e^(m_s - M), 0 for a split without keys
  __shared__ float lf[MAX_SPLITS];  // l_s * e^(m_s - M)
  __shared__ float wmax[HD / 64];
  const int M = G * R;
  // query-major numbering: workgroup m * Hkv + g.  The split kernel's grid
  // (Hkv, splits) puts every split of KV head g on XCD (g + Hkv s) % 8, g % 8
  // when Hkv % 8 == 0 (workgroups are dealt to the eight XCDs round robin in
  // launch order), and so does this numbering: the partial results are read
  // from the L2 of the XCD that wrote them
  const int g = static_cast<int>(blockIdx.x) % Hkv, m = static_cast<int>(blockIdx.x) / Hkv;
  const int d = threadIdx.x;
  auto stat = [&](int s) { return (static_cast<int64_t>(s) * Hkv + g) * M + m; };
  float pre[PRE];
#pragma unroll
  for (int j = 0; j < PRE; ++j) pre[j] = j < splits ? part_o[stat(j) * HD + d] : 0.f;
  float mx = -__builtin_inff();
  for (int s = d; s < splits; s += HD) mx = fmaxf(mx, part_ml[stat(s) * 2]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((d & 63) == 0) wmax[d >> 6] = mx;
  __syncthreads();
  mx = wmax[0];
#pragma unroll
  for (int i = 1; i < HD / 64; ++i) mx = fmaxf(mx, wmax[i]);
  for (int s = d; s < splits; s += HD) {
    const float ms = part_ml[stat(s) * 2];
    const float e = ms == -__builtin_inff() ? 0.f : expf(ms - mx);
    f[s] = e;
    lf[s] = part_ml[stat(s) * 2 + 1] * e;
  }
  __syncthreads();
  float l = 0.f, acc = 0.f;
#pragma unroll
  for (int j = 0; j < PRE; ++j)
    if (j < splits && f[j] != 0.f) {
      l += lf[j];
      acc += pre[j] * f[j];
    }
  for (int s0 = PRE; s0 < splits; s0 += 16) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = s0 + j < splits ? part_o[stat(s0 + j) * HD + d] : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (s0 + j < splits && f[s0 + j] != 0.f) {
        l += lf[s0 + j];
        acc += v[j] * f[s0 + j];
      }
  }
  const int r = m % R, hq = g * G + m / R;
  out[(static_cast<int64_t>(r) * Hq + hq) * HD + d] = acc / l;
}

__global__ void __launch_bounds__(64)
tree_commit_kernel(uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, int64_t cache_len, int ctx_len,
                   const uint16_t* __restrict__ ks, const uint16_t* __restrict__ vs, int scr_len,
                   const int32_t* __restrict__ path, int n_path, int D) {
  const int g = blockIdx.x, i = blockIdx.y;
  const int slot = path[i];
  if (slot < 0 || slot >= scr_len) return;  // an invalid slot index leaves its position unchanged
  const int64_t src = (static_cast<int64_t>(g) * scr_len + slot) * D;
  const int64_t dst = (static_cast<int64_t>(g) * cache_len + ctx_len + i) * D;
  for (int c = threadIdx.x; c < D / 8; c += 64) {
    *reinterpret_cast<u32x4*>(kc + dst + c * 8) = *reinterpret_cast<const u32x4*>(ks + src + c * 8);
    *reinterpret_cast<u32x4*>(vc + dst + c * 8) = *reinterpret_cast<const u32x4*>(vs + src + c * 8);
  }
}

// context sub-blocks per split: enough splits to give the device about two
// workgroups per CU, at least one sub-block each (more splits than the
// resident slots, two 64 KB workgroups per CU, add a second round)
int blocks_per_split(int ctx_len, int Hkv) {
  const int nblk = (ctx_len + BKEYS - 1) / BKEYS;
  const int target = (256 + Hkv - 1) / Hkv;  // splits per KV head (<= 256)
  int nb = (nblk + target - 1) / target;
  return nb < 1 ? 1 : nb;
}

struct Plan {
  int nb, ctx_splits, splits, M;
};

Plan plan_for(int R, int Hq, int Hkv, int ctx_len) {
  Plan p;
  p.nb = blocks_per_split(ctx_len, Hkv);
  const int nblk = (ctx_len + BKEYS - 1) / BKEYS;
  p.ctx_splits = (nblk + p.nb - 1) / p.nb;
  p.splits = p.ctx_splits + 1;
  p.M = (Hq / Hkv) * R;
  return p;
}

}  // namespace

extern "C" size_t tree_attention_rows_workspace_bytes(int R, int Hq, int Hkv, int ctx_len) {
  if (R < 1 || Hq < 1 || Hkv < 1 || ctx_len < 0 || Hq % Hkv != 0) return 0;
  const Plan p = plan_for(R, Hq, Hkv, ctx_len);
  return static_cast<size_t>(p.splits) * Hkv * p.M * (HD + 2) * sizeof(float);
}

extern "C" int tree_attention_rows(const float* q, int R, int Hq, int D, const uint16_t* k_cache,
                                   const uint16_t* v_cache, int64_t cache_len, int ctx_len,
                                   const uint16_t* k_scr, const uint16_t* v_scr, int scr_len,
                                   const int32_t* parent, int Hkv, float scale, float* out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k_scr || !v_scr || !out) return VS_ERR_NULL;
  if (ctx_len > 0 && (!k_cache || !v_cache)) return VS_ERR_NULL;
  if (R > 1 && !parent) return VS_ERR_NULL;
  if (D != HD) return VS_ERR_UNSUPPORTED;
  if (R < 1 || R > MAX_ROWS || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return VS_ERR_SHAPE;
  if ((Hq / Hkv) * R > MAX_QUERIES) return VS_ERR_SHAPE;
  if (ctx_len < 0 || cache_len < ctx_len || scr_len < R) return VS_ERR_SHAPE;
  if (!__builtin_isfinite(scale)) return VS_ERR_PARAM;
  if (!vs::aligned16(q) || !vs::aligned16(k_scr) || !vs::aligned16(v_scr) ||
      (ctx_len > 0 && (!vs::aligned16(k_cache) || !vs::aligned16(v_cache))))
    return VS_ERR_ALIGN;
  const size_t need = tree_attention_rows_workspace_bytes(R, Hq, Hkv, ctx_len);
  if (!workspace || workspace_bytes < need) return VS_ERR_WORKSPACE;
  if (!vs::aligned16(workspace)) return VS_ERR_ALIGN;
  const Plan p = plan_for(R, Hq, Hkv, ctx_len);
  if (p.splits > MAX_SPLITS) return VS_ERR_SHAPE;  // not reached: plan_for keeps splits <= 257
  Args a;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.cache_len = cache_len;
  a.ctx_len = ctx_len;
  a.ks = k_scr;
  a.vs = v_scr;
  a.scr_len = scr_len;
  a.parent = parent;
  a.R = R;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.scale = scale;
  a.NB = p.nb;
  a.ctx_splits = p.ctx_splits;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = a.part_o + static_cast<size_t>(p.splits) * Hkv * p.M * HD;
  // one 16-query tile per wave, the query tiles spread over grid.z
  const int mt = (p.M + 15) / 16;  // <= 16 (M <= 256)
  const dim3 grid(Hkv, p.splits, (mt + WAVES - 1) / WAVES), block(64 * WAVES);
  tree_attention_split_kernel<1, true><<<grid, block, 0, stream>>>(a);
  int st = vs::check_launch();
  if (st != VS_OK) return st;
  tree_attention_combine_kernel<<<dim3(Hkv * p.M), dim3(HD), 0, stream>>>(
      a.part_o, a.part_ml, p.splits, Hkv, a.G, R, Hq, out);
  return vs::check_launch();
}

extern "C" int tree_commit_kv(uint16_t* k_cache, uint16_t* v_cache, int64_t cache_len, int ctx_len,
                              const uint16_t* k_scr, const uint16_t* v_scr, int scr_len,
                              const int32_t* path, int n_path, int Hkv, int D, hipStream_t stream) {
  if (!k_cache || !v_cache || !k_scr || !v_scr) return VS_ERR_NULL;
  if (n_path > 0 && !path) return VS_ERR_NULL;
  if (Hkv < 1 || D < 8 || D % 8 != 0 || n_path < 0 || n_path > MAX_ROWS || scr_len < 1) return VS_ERR_SHAPE;
  if (ctx_len < 0 || static_cast<int64_t>(ctx_len) + n_path > cache_len) return VS_ERR_SHAPE;
  if (!vs::aligned16(k_cache) || !vs::aligned16(v_cache) || !vs::aligned16(k_scr) || !vs::aligned16(v_scr))
    return VS_ERR_ALIGN;
  if (n_path == 0) return VS_OK;
  tree_commit_kernel<<<dim3(Hkv, n_path), dim3(64), 0, stream>>>(k_cache, v_cache, cache_len, ctx_len, k_scr,
                                                                 v_scr, scr_len, path, n_path, D);
  return vs::check_launch();
}
