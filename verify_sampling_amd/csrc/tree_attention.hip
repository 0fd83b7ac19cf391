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
//  * values: the probabilities, split exactly into three bf16 planes in LDS
//    (the A operand), times V transposed into LDS (the B operand);
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
constexpr int WAVES = 4;
constexpr int KSTEPS = HD / 32;     // MFMA k-steps over the head dimension
constexpr int NT_S = BKEYS / 16;    // key tiles of a sub-block
constexpr int NT_O = HD / 16;       // dimension tiles of the output
constexpr int PSTR = BKEYS + 8;     // LDS row stride (bf16) of the probability planes
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

// max / sum over the 16 lanes of a row group (lanes l with equal l / 16),
// always in the same butterfly order
__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// The scratch slots row `row` attends to, as a bit mask (bit s = slot s).
__device__ __forceinline__ uint64_t ancestor_mask(const int32_t* __restrict__ parent, int row) {
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

// MTW: 16-query tiles per wave (M = G * R <= 64 * WAVES * MTW)
template <int MTW>
__global__ void __launch_bounds__(64 * WAVES)
tree_attention_split_kernel(Args a) {
  __shared__ __align__(16) uint16_t pl[WAVES][MTW][3][16 * PSTR];  // probability planes, per wave
  __shared__ __align__(16) uint16_t vt[HD * VSTR];                 // V of the sub-block, transposed
  const int lane = threadIdx.x & 63;
  const int w = vs::wave_index();
  const int g = blockIdx.x;                 // KV head
  const int split = blockIdx.y;
  const bool scratch = split == a.ctx_splits;
  const int M = a.G * a.R;
  const int col = lane & 15, grp = lane >> 4;

  // this wave's query tiles: mt = w + WAVES * i; per lane, the scratch
  // slots visible to the query row of each of its C elements (4 per tile;
  // padding rows past M see slot 0 only, and their results are dropped)
  uint64_t anc[MTW][4];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = (w + WAVES * i) * 16 + 4 * grp + e;
      anc[i][e] = (scratch && m < M) ? ancestor_mask(a.parent, m % a.R) : 1ull;
    }

  f32x4 o[MTW][NT_O];
  float rm[MTW][4], rl[MTW][4];
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
#pragma unroll
    for (int t = 0; t < NT_O; ++t) o[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rm[i][e] = -__builtin_inff();
      rl[i][e] = 0.f;
    }
  }

  const uint16_t* kbase = scratch ? a.ks + static_cast<int64_t>(g) * a.scr_len * HD
                                  : a.kc + static_cast<int64_t>(g) * a.cache_len * HD;
  const uint16_t* vbase = scratch ? a.vs + static_cast<int64_t>(g) * a.scr_len * HD
                                  : a.vc + static_cast<int64_t>(g) * a.cache_len * HD;
  const int nsub = scratch ? 1 : a.NB;
  for (int sb = 0; sb < nsub; ++sb) {
    // keys of this sub-block: positions p0 .. p0 + 63 below nkeys
    const int p0 = scratch ? 0 : (split * a.NB + sb) * BKEYS;
    const int nkeys = scratch ? a.R : a.ctx_len;
    if (!scratch && p0 >= nkeys) break;  // uniform over the workgroup

    // V of the sub-block into LDS, transposed ([dim][key]); keys past the
    // end are zero (their probabilities are zero, and 0 * garbage could be NaN)
    __syncthreads();  // the previous sub-block's vt has been read
    for (int c = threadIdx.x; c < BKEYS * HD / 8; c += 64 * WAVES) {
      const int key = c / (HD / 8), d0 = (c % (HD / 8)) * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (p0 + key < nkeys) v = *reinterpret_cast<const u32x4*>(vbase + static_cast<int64_t>(p0 + key) * HD + d0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vt[(d0 + 2 * j) * VSTR + key] = static_cast<uint16_t>(v[j] & 0xffffu);
        vt[(d0 + 2 * j + 1) * VSTR + key] = static_cast<uint16_t>(v[j] >> 16);
      }
    }

    // scores: S[query][key] for this wave's tiles
    f32x4 s[MTW][NT_S];
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int t = 0; t < NT_S; ++t) s[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int d = ks * 32 + grp * 8;
      u32x4 kb[NT_S];
#pragma unroll
      for (int t = 0; t < NT_S; ++t) {
        const int key = p0 + t * 16 + col;
        kb[t] = key < nkeys ? *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(key) * HD + d)
                            : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < MTW; ++i) {
        const int m = (w + WAVES * i) * 16 + col;  // A operand: query row col of the tile
        float x[8];
        if (m < M) {
          const int r = m % a.R, hq = g * a.G + m / a.R;
          const float* src = a.q + (static_cast<int64_t>(r) * a.Hq + hq) * HD + d;
          const float4 x0 = *reinterpret_cast<const float4*>(src);
          const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
          x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
          x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = 0.f;
        }
        u32x4 hi, mid, lo;
        split3(x, hi, mid, lo);
#pragma unroll
        for (int t = 0; t < NT_S; ++t) {
          s[i][t] = mfma(hi, kb[t], s[i][t]);
          s[i][t] = mfma(mid, kb[t], s[i][t]);
          s[i][t] = mfma(lo, kb[t], s[i][t]);
        }
      }
    }

    // online softmax over the sub-block; probabilities into this wave's planes
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      float alpha[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float bm = -__builtin_inff();
#pragma unroll
        for (int t = 0; t < NT_S; ++t) {
          const int key = t * 16 + col;  // within the sub-block
          const bool ok = scratch ? (key < a.R && ((anc[i][e] >> key) & 1ull)) : (p0 + key < nkeys);
          s[i][t][e] = ok ? s[i][t][e] * a.scale : -__builtin_inff();
          bm = fmaxf(bm, s[i][t][e]);
        }
        bm = group16_max(bm);  // every row sees at least one key of every sub-block
        const float mn = fmaxf(rm[i][e], bm);
        alpha[e] = expf(rm[i][e] - mn);  // 0 on the first sub-block
        rm[i][e] = mn;
        float ps = 0.f;
#pragma unroll
        for (int t = 0; t < NT_S; ++t) {
          const float p = expf(s[i][t][e] - mn);  // 0 for masked keys
          ps += p;
          uint16_t h, md, l;
          split3_one(p, h, md, l);
          const int off = (4 * grp + e) * PSTR + t * 16 + col;
          pl[w][i][0][off] = h;
          pl[w][i][1][off] = md;
          pl[w][i][2][off] = l;
        }
        rl[i][e] = rl[i][e] * alpha[e] + group16_sum(ps);
      }
      // rescale the running output rows (C layout: element e is row 4 grp + e)
#pragma unroll
      for (int t = 0; t < NT_O; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[i][t][e] *= alpha[e];
    }
    __syncthreads();  // vt written by all waves; this wave's planes written

    // output += P V: A = probability planes (query col, keys 8 grp ..), B = V^T
#pragma unroll
    for (int kk = 0; kk < BKEYS / 32; ++kk) {
      const int k0 = kk * 32 + grp * 8;
      u32x4 vb[NT_O];
#pragma unroll
      for (int t = 0; t < NT_O; ++t)
        vb[t] = *reinterpret_cast<const u32x4*>(&vt[(t * 16 + col) * VSTR + k0]);
#pragma unroll
      for (int i = 0; i < MTW; ++i) {
        const u32x4 ph = *reinterpret_cast<const u32x4*>(&pl[w][i][0][col * PSTR + k0]);
        const u32x4 pm = *reinterpret_cast<const u32x4*>(&pl[w][i][1][col * PSTR + k0]);
        const u32x4 pq = *reinterpret_cast<const u32x4*>(&pl[w][i][2][col * PSTR + k0]);
#pragma unroll
        for (int t = 0; t < NT_O; ++t) {
          o[i][t] = mfma(ph, vb[t], o[i][t]);
          o[i][t] = mfma(pm, vb[t], o[i][t]);
          o[i][t] = mfma(pq, vb[t], o[i][t]);
        }
      }
    }
  }

  // partial results of this split: rows of real queries only
  const int64_t base = (static_cast<int64_t>(split) * a.Hkv + g) * M;
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = (w + WAVES * i) * 16 + 4 * grp + e;
      if (m >= M) continue;
      float* dst = a.part_o + (base + m) * HD;
#pragma unroll
      for (int t = 0; t < NT_O; ++t) dst[t * 16 + col] = o[i][t][e];
      if (col == 0) {
        a.part_ml[(base + m) * 2] = rm[i][e];
        a.part_ml[(base + m) * 2 + 1] = rl[i][e];
      }
    }
}

// out[r][hq][d] from the splits' partial results, merged in split order.
__global__ void __launch_bounds__(HD)
tree_attention_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                              int splits, int Hkv, int G, int R, int Hq, float* __restrict__ out) {
  const int M = G * R;
  const int gm = blockIdx.x;  // g * M + m
  const int g = gm / M, m = gm % M;
  const int d = threadIdx.x;
  float mx = -__builtin_inff();
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, part_ml[((static_cast<int64_t>(s) * Hkv + g) * M + m) * 2]);
  float l = 0.f, acc = 0.f;
  for (int s = 0; s < splits; ++s) {
    const int64_t idx = (static_cast<int64_t>(s) * Hkv + g) * M + m;
    const float ms = part_ml[idx * 2];
    if (ms == -__builtin_inff()) continue;  // a split with no key for this row
    const float f = expf(ms - mx);
    l += part_ml[idx * 2 + 1] * f;
    acc += part_o[idx * HD + d] * f;
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
// workgroups per CU, at least one sub-block each
int blocks_per_split(int ctx_len, int Hkv) {
  const int nblk = (ctx_len + BKEYS - 1) / BKEYS;
  const int target = (512 + Hkv - 1) / Hkv;  // splits per KV head
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
  const dim3 grid(Hkv, p.splits), block(64 * WAVES);
  const int mt = (p.M + 15) / 16;
  if (mt <= WAVES) tree_attention_split_kernel<1><<<grid, block, 0, stream>>>(a);
  else if (mt <= 2 * WAVES) tree_attention_split_kernel<2><<<grid, block, 0, stream>>>(a);
  else tree_attention_split_kernel<4><<<grid, block, 0, stream>>>(a);
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
