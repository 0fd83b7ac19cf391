// verify_gemv_rows: the multi-row verify projection on gfx950 matrix cores.
//
// "Speculative decoding on RDNA", §01: a verify pass reads every weight once
// for all k + 1 rows; §02: the multi-row projections sum in exactly the
// single-row decode order.
//
// Design (MI355X):
//  * The weights are the only large operand, so the kernel is an HBM stream:
//    each lane issues 16-byte loads of 8 consecutive bf16 weights, and every
//    loaded weight is used for all R rows before it is dropped.
//  * The R activation rows ride in the N dimension of a 16x16x32 bf16 MFMA
//    (weights are the A operand, 16 output rows x 32 k; activations are B).
//    R <= 16 uses one 16-column tile, R <= 24 two.  MFMA keeps the cost of an
//    extra row near zero: at R = 24 an fp32 FMA loop would need ~24 VALU ops
//    per weight, more than the VALU can issue at HBM speed.
//  * fp32 activations are kept exact: each x is split into three bf16 pieces
//    hi + mid + lo == x (truncation leaves at most 16, then 8 significant
//    bits, each exactly representable), so every bf16 x bf16 product is
//    exact and the MFMA accumulates in fp32.
//  * Order invariance: output element (n, r) only ever combines W[n][:] with
//    X[r][:] (MFMA computes each output element from its own row and column),
//    the k-blocks each wave owns and their order depend only on K, and the
//    per-wave partial sums are added in wave order.  None of this depends on
//    R or on the column a row lands in, so row r of an R-row call equals the
//    1-row call on X[r] bit for bit.
//  * Workgroup = `splits` wavefronts over T 16-row tiles; wave w owns
//    k-blocks [w*nkb/splits, (w+1)*nkb/splits).  Partial sums meet in LDS.

#include "vs_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int KBLK = 32;   // k per MFMA step
constexpr int TILE = 16;   // weight rows per tile

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bitsf(uint32_t b) { return __builtin_bit_cast(float, b); }

// Splits 8 fp32 values into three bf16x8 planes with x == hi + mid + lo exactly.
__device__ __forceinline__ void split3(const float (&x)[8], u32x4& hi, u32x4& mid, u32x4& lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t h0 = fbits(x[2 * p]) & 0xffff0000u, h1 = fbits(x[2 * p + 1]) & 0xffff0000u;
    float r0 = x[2 * p] - bitsf(h0), r1 = x[2 * p + 1] - bitsf(h1);
    uint32_t m0 = fbits(r0) & 0xffff0000u, m1 = fbits(r1) & 0xffff0000u;
    float s0 = r0 - bitsf(m0), s1 = r1 - bitsf(m1);
    hi[p] = (h0 >> 16) | h1;
    mid[p] = (m0 >> 16) | m1;
    lo[p] = (fbits(s0) >> 16) | (fbits(s1) & 0xffff0000u);
  }
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One pipeline stage: the weights of U k-blocks for T row tiles, and the
// activations of those k-blocks for CT column tiles.
template <int T, int U, int CT>
struct Stage {
  u32x4 w[U][T];
  float x[U][CT][8];
};

template <int T, int U, int CT>
__device__ __forceinline__ void load_stage(Stage<T, U, CT>& st, int kb, int kb1, int K, int g,
                                           const uint16_t* const (&wrow)[T],
                                           const float* const (&xrow)[CT], const bool (&xon)[CT]) {
  // activations first: memory returns in issue order, so the split of this
  // stage's activations can start while its weights are still arriving
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = (kb + u) * KBLK + g * 8;
    const bool ok = (kb + u < kb1) && (k < K);  // K % 8 == 0: k < K covers all 8 values
    const int64_t off = static_cast<int64_t>(kb + u) * KBLK;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      if (ok && xon[c]) {
        const float4 a = *reinterpret_cast<const float4*>(xrow[c] + off);
        const float4 b = *reinterpret_cast<const float4*>(xrow[c] + off + 4);
        st.x[u][c][0] = a.x; st.x[u][c][1] = a.y; st.x[u][c][2] = a.z; st.x[u][c][3] = a.w;
        st.x[u][c][4] = b.x; st.x[u][c][5] = b.y; st.x[u][c][6] = b.z; st.x[u][c][7] = b.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) st.x[u][c][e] = 0.f;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = (kb + u) * KBLK + g * 8;
    const bool ok = (kb + u < kb1) && (k < K);
    const int64_t off = static_cast<int64_t>(kb + u) * KBLK;
#pragma unroll
    for (int t = 0; t < T; ++t)
      st.w[u][t] = ok ? *reinterpret_cast<const u32x4*>(wrow[t] + off) : u32x4{0u, 0u, 0u, 0u};
  }
}

// Accumulates the stage's k-blocks in increasing k order: per k-block the
// hi, mid and lo products, in that order.
template <int T, int U, int CT>
__device__ __forceinline__ void compute_stage(const Stage<T, U, CT>& st, int kb, int kb1,
                                              f32x4 (&acc)[T][CT]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (kb + u >= kb1) break;  // uniform across the wave
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      u32x4 hi, mid, lo;
      split3(st.x[u][c], hi, mid, lo);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        acc[t][c] = mfma(st.w[u][t], hi, acc[t][c]);
        acc[t][c] = mfma(st.w[u][t], mid, acc[t][c]);
        acc[t][c] = mfma(st.w[u][t], lo, acc[t][c]);
      }
    }
  }
}

// T: 16-row weight tiles per wave (the activations are loaded and split once
// for all T); U: k-blocks per stage; CT: 16-column activation tiles; PIPE:
// load stage s+1 while computing stage s.  None of these changes the order in
// which a row is summed.
template <int T, int U, int CT, bool PIPE, bool XF = false>
__global__ void __launch_bounds__(1024)
gemv_rows_kernel(const uint16_t* __restrict__ W, int64_t ldw, int N, int K,
                 const float* __restrict__ X, int64_t ldx, int R,
                 float* __restrict__ Y, int64_t ldy, int nkb, int splits) {
  extern __shared__ float red[];  // [splits][T][CT][4][64 lanes]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;     // which 8-wide k slice of the 32-wide block
  const int col = lane & 15;   // A: weight row within the tile; B: activation row
  const int n0 = blockIdx.x * TILE * T;

  const uint16_t* wrow[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    int wr = n0 + t * TILE + col;
    if (wr >= N) wr = N - 1;  // ragged tile: load a valid row, discard its results
    wrow[t] = W + static_cast<int64_t>(wr) * ldw + g * 8;
  }
  const float* xrow[CT];
  bool xon[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int r = c * 16 + col;
    xon[c] = r < R;
    xrow[c] = X + static_cast<int64_t>(xon[c] ? r : 0) * ldx + g * 8;
  }

  const int kb0 = static_cast<int>((static_cast<int64_t>(wave) * nkb) / splits);
  const int kb1 = static_cast<int>((static_cast<int64_t>(wave + 1) * nkb) / splits);

  f32x4 acc[T][CT];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (PIPE) {
    Stage<T, U, CT> sa, sb;
    load_stage(sa, kb0, kb1, K, g, wrow, xrow, xon);
    for (int kb = kb0; kb < kb1; kb += 2 * U) {
      if (kb + U < kb1) load_stage(sb, kb + U, kb1, K, g, wrow, xrow, xon);
      compute_stage(sa, kb, kb1, acc);
      if (kb + U >= kb1) break;
      if (kb + 2 * U < kb1) load_stage(sa, kb + 2 * U, kb1, K, g, wrow, xrow, xon);
      compute_stage(sb, kb + U, kb1, acc);
    }
  } else if (XF) {
    // activations of the stage first, then its weights (see load_stage)
    for (int kb = kb0; kb < kb1; kb += U) {
      Stage<T, U, CT> st;
      load_stage(st, kb, kb1, K, g, wrow, xrow, xon);
      compute_stage(st, kb, kb1, acc);
    }
  } else {
    // weights of U k-blocks in flight; each k-block's activations are loaded
    // just before use, which keeps the register count at full occupancy
    for (int kb = kb0; kb < kb1; kb += U) {
      u32x4 wv[U][T];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = (kb + u) * KBLK + g * 8;
        const bool ok = (kb + u < kb1) && (k < K);
        const int64_t off = static_cast<int64_t>(kb + u) * KBLK;
#pragma unroll
        for (int t = 0; t < T; ++t)
          wv[u][t] = ok ? *reinterpret_cast<const u32x4*>(wrow[t] + off) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (kb + u >= kb1) break;  // uniform across the wave
        const int k = (kb + u) * KBLK + g * 8;
        const int64_t off = static_cast<int64_t>(kb + u) * KBLK;
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          float xv[8];
          if (xon[c] && k < K) {
            const float4 a = *reinterpret_cast<const float4*>(xrow[c] + off);
            const float4 b = *reinterpret_cast<const float4*>(xrow[c] + off + 4);
            xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
            xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) xv[e] = 0.f;
          }
          u32x4 hi, mid, lo;
          split3(xv, hi, mid, lo);
#pragma unroll
          for (int t = 0; t < T; ++t) {
            acc[t][c] = mfma(wv[u][t], hi, acc[t][c]);
            acc[t][c] = mfma(wv[u][t], mid, acc[t][c]);
            acc[t][c] = mfma(wv[u][t], lo, acc[t][c]);
          }
        }
      }
    }
  }

  // Partial sums of all waves meet in LDS and are added in wave order.
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        red[(((wave * T + t) * CT + c) * 4 + e) * 64 + lane] = acc[t][c][e];
  __syncthreads();
  const int per_wave = T * CT * 256;
  for (int idx = threadIdx.x; idx < per_wave; idx += blockDim.x) {
    float s = red[idx];
    for (int w = 1; w < splits; ++w) s += red[w * per_wave + idx];
    const int l = idx & 63;
    const int e = (idx >> 6) & 3;
    const int c = (idx >> 8) % CT;
    const int t = (idx >> 8) / CT;
    // MFMA 16x16 output layout: lane l, element e holds row 4*(l/16)+e of the
    // tile (the weight row) and column l%16 (the activation row).
    const int n = n0 + t * TILE + 4 * (l >> 4) + e;
    const int r = c * 16 + (l & 15);
    if (n < N && r < R) Y[static_cast<int64_t>(r) * ldy + n] = s;
  }
}

// Waves per workgroup (the k-split): a function of N and K alone, so that
// the summation order of a row does not change with R.  Wide matrices (many
// row tiles) do best with few, long waves; narrower ones split K further
// for parallelism.  Chosen by a sweep on MI355X.
int splits_for(int N, int K) {
  const int nkb = (K + KBLK - 1) / KBLK;
  int s = (N >= 16384) ? (nkb + 31) / 32 : (nkb + 15) / 16;
  if (s < 1) s = 1;
  if (s > (N >= 16384 ? 16 : 8)) s = (N >= 16384 ? 16 : 8);
  return s;
}

}  // namespace

extern "C" int verify_gemv_rows(const uint16_t* W, int64_t ldw, int N, int K, const float* X,
                                int64_t ldx, int R, float* Y, int64_t ldy, hipStream_t stream) {
  if (!W || !X || !Y) return VS_ERR_NULL;
  if (N < 1 || K < 1 || R < 1 || R > VS_MAX_ROWS) return VS_ERR_SHAPE;
  if (K % 8 != 0 || ldw < K || ldx < K || ldy < N) return VS_ERR_SHAPE;
  if (ldw % 8 != 0 || ldx % 4 != 0 || !vs::aligned16(W) || !vs::aligned16(X)) return VS_ERR_ALIGN;
  if (static_cast<int64_t>(N) > (int64_t{1} << 31) - TILE) return VS_ERR_SHAPE;

  const int nkb = (K + KBLK - 1) / KBLK;
  const int splits = splits_for(N, K);
  const dim3 block(64 * splits);
  // Tile shape by matrix shape and R (it never changes a row's summation
  // order): taller matrices take more row tiles per wave, which divides the
  // activation traffic and the splitting work per weight; "activations
  // first" issues a stage's activation loads ahead of its weights so that
  // their split overlaps the weight latency.  Chosen by a sweep on MI355X.
  auto launch = [&](auto kernel, int T, int CT) {
    const dim3 grid((N + TILE * T - 1) / (TILE * T));
    const size_t shm = static_cast<size_t>(splits) * T * CT * 256 * sizeof(float);
    kernel<<<grid, block, shm, stream>>>(W, ldw, N, K, X, ldx, R, Y, ldy, nkb, splits);
  };
  if (R <= 16) {
    if (N >= 65536 && R > 8) launch(gemv_rows_kernel<4, 1, 1, false, true>, 4, 1);
    else if (N >= 65536) launch(gemv_rows_kernel<2, 4, 1, false, true>, 2, 1);
    else if (N >= 16384 && R > 8) launch(gemv_rows_kernel<2, 2, 1, false, false>, 2, 1);
    else if (N >= 6144) launch(gemv_rows_kernel<2, 2, 1, false, true>, 2, 1);
    else launch(gemv_rows_kernel<1, 4, 1, false, true>, 1, 1);
  } else {
    if (N >= 65536) launch(gemv_rows_kernel<4, 1, 2, false, false>, 4, 2);
    else if (N >= 6144) launch(gemv_rows_kernel<2, 2, 2, false, false>, 2, 2);
    else launch(gemv_rows_kernel<1, 2, 2, true, false>, 1, 2);
  }
  return vs::check_launch();
}
