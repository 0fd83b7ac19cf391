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
//  * K is cut into `splits` partitions [s*nkb/splits, (s+1)*nkb/splits) of
//    32-wide k-blocks, a function of N and K alone.  Each partition is
//    accumulated from zero in increasing k order, and the partition sums
//    are added left to right.  Every kernel below follows exactly this
//    order, so they all give the same bits and may be chosen per R.
//  * Row-block kernels: workgroup = `splits` wavefronts over T 16-row tiles;
//    wave w owns partition w; partial sums meet in LDS.  Every wave loads
//    and splits the activations of its partition itself.  The MFMA operand
//    layout wants 16 rows x 64 bytes per load instruction, which HBM serves
//    worse than long row runs, so the staged variant loads 8 rows x 128
//    bytes per instruction (branch-free, one stage ahead) and restages each
//    stage through the wave's own LDS region into the operand layout.  The
//    plain variant (operands loaded in place) covers the shapes the staged
//    one does not (K % 32 != 0, short partitions, more than 8 waves).
//  * Shared-activation kernels (many rows): a workgroup of P wavefronts
//    along N loads each activation tile once, splits it once into the three
//    bf16 planes in LDS, and all P waves read their MFMA operand from there.
//    This divides the activation traffic per weight byte by P, which is what
//    makes a row-block pass slow down with R.  Each workgroup takes one
//    partition (grid.y) and writes its partial sums to a caller workspace,
//    which a second small kernel adds in partition order; the staged form
//    loads its weights as the staged row-block kernel does.  Where the
//    staged kernels cannot run, an older form loads weights in the operand
//    layout and may instead walk all of K per wave, adding its partition sums
//    in registers (very wide matrices).

#include <cmath>
#include <type_traits>

#include "vs_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int KBLK = 32;   // k per MFMA step
constexpr int TILE = 16;   // weight rows per tile

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bitsf(uint32_t b) { return __builtin_bit_cast(float, b); }

// x minus its top plane, the part the lower planes hold: exact for finite
// x; 0 for x = +-inf (whose difference with itself would be NaN), so that an
// infinite activation contributes hi * w = +-inf (NaN for w = 0) as its term
// of the sum does.  A NaN activation stays NaN through its top plane or its
// residual.
__device__ __forceinline__ float residual(float x, uint32_t h) {
  const float r = x - bitsf(h);
  return __builtin_isinf(x) ? 0.f : r;
}

// Splits 8 fp32 values into three bf16x8 planes with x == hi + mid + lo
// exactly (finite x; an infinite one is hi alone, see residual).
__device__ __forceinline__ void split3(const float (&x)[8], u32x4& hi, u32x4& mid, u32x4& lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t h0 = fbits(x[2 * p]) & 0xffff0000u, h1 = fbits(x[2 * p + 1]) & 0xffff0000u;
    float r0 = residual(x[2 * p], h0), r1 = residual(x[2 * p + 1], h1);
    uint32_t m0 = fbits(r0) & 0xffff0000u, m1 = fbits(r1) & 0xffff0000u;
    float s0 = r0 - bitsf(m0), s1 = r1 - bitsf(m1);
    hi[p] = (h0 >> 16) | h1;
    mid[p] = (m0 >> 16) | m1;
    lo[p] = (fbits(s0) >> 16) | (fbits(s1) & 0xffff0000u);
  }
}

// Weight loads are marked non-temporal: every weight is read once per call,
// and keeping the stream from displacing cached lines (the activations, which
// every workgroup re-reads) raised the loads-only streaming rate on MI355X by
// 4-12% (LM head 5.9 -> 6.6 TB/s).
__device__ __forceinline__ u32x4 load_weights(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Splits 4 fp32 values as split3 does, into two dwords (four bf16) per plane.
__device__ __forceinline__ void split3x4(float4 x, uint2& hi, uint2& mid, uint2& lo) {
  const float v[4] = {x.x, x.y, x.z, x.w};
  uint32_t h[2], m[2], l[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    uint32_t h0 = fbits(v[2 * p]) & 0xffff0000u, h1 = fbits(v[2 * p + 1]) & 0xffff0000u;
    float r0 = residual(v[2 * p], h0), r1 = residual(v[2 * p + 1], h1);
    uint32_t m0 = fbits(r0) & 0xffff0000u, m1 = fbits(r1) & 0xffff0000u;
    float s0 = r0 - bitsf(m0), s1 = r1 - bitsf(m1);
    h[p] = (h0 >> 16) | h1;
    m[p] = (m0 >> 16) | m1;
    l[p] = (fbits(s0) >> 16) | (fbits(s1) & 0xffff0000u);
  }
  hi = uint2{h[0], h[1]};
  mid = uint2{m[0], m[1]};
  lo = uint2{l[0], l[1]};
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
      st.w[u][t] = ok ? load_weights(wrow[t] + off) : u32x4{0u, 0u, 0u, 0u};
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
// for all T); U: k-blocks per stage; CT: 16-column activation tiles; XF: a
// stage's activations are loaded ahead of its weights.  None of these changes
// the order in which a row is summed.
template <int T, int U, int CT, bool XF>
__global__ void __launch_bounds__(1024)
gemv_rows_kernel(const uint16_t* __restrict__ W, int64_t ldw, int N, int K,
                 const float* __restrict__ X, int64_t ldx, int R,
                 float* __restrict__ Y, int64_t ldy, int nkb, int splits) {
  extern __shared__ float red[];  // [splits][T][CT][4][64 lanes]
  const int lane = threadIdx.x & 63;
  const int wave = vs::wave_index();
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

  if (XF) {
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
          wv[u][t] = ok ? load_weights(wrow[t] + off) : u32x4{0u, 0u, 0u, 0u};
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

// Staged row-block kernel: stage = U k-blocks of the wave's T*16 rows, loaded
// as RPI rows x RB bytes per instruction (row runs instead of the operand
// layout's 16 x 64 bytes), written to the wave's LDS region (rows padded by
// 16 bytes so that the operand reads spread over the banks) and read back as
// MFMA A operands.  Loads carry no per-lane guards, so the next stage stays
// in flight while this one is computed: a stage past the partition's end
// re-reads the range's last k-blocks and computes nothing.  Wave w owns PPW
// consecutive partitions (one accumulator set each), so the partition count
// can exceed the wave count; the partition sums are added in partition
// order, as in gemv_rows_kernel.  Requires K % 32 == 0, every partition >= U
// k-blocks, and <= LB threads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int T, int U, int CT, int XL>
struct RunStage {
  u32x4 w[T * TILE * U * 64 / 1024];  // this lane's 16-byte pieces of the stage
  // activations: XL, one 16-byte piece per load instruction (at most
  // CT * 16 rows x U k-blocks x 128 bytes); direct, the lane's own column
  float4 x[XL > 0 ? XL : U * CT * 2];
};

template <int T, int U, int CT, int LB, int PPW, int XL, bool XP = false>
__global__ void __launch_bounds__(LB)
gemv_rows_staged_kernel(const uint16_t* __restrict__ W, int64_t ldw, int N, int K,
                        const float* __restrict__ X, int64_t ldx, int R,
                        float* __restrict__ Y, int64_t ldy, int nkb, int splits) {
  extern __shared__ float red[];  // stage buffers during the loop, then the reduction
  constexpr int RB = U * 64;      // bytes of one row per stage
  constexpr int RS = RB + 16;     // LDS row stride
  constexpr int LPR = RB / 16;    // lanes per row in one load
  constexpr int RPI = 64 / LPR;   // rows per load instruction
  constexpr int NI = T * TILE / RPI;
  static_assert(64 % LPR == 0 && (T * TILE) % RPI == 0, "stage shape");
  const int lane = threadIdx.x & 63;
  const int wave = vs::wave_index();
  const int g = lane >> 4;
  const int col = lane & 15;
  const int n0 = blockIdx.x * TILE * T;
  // XL: activations go through LDS as well (XB bytes per wave after the
  // weights), loaded as whole 128-byte rows of a k-block
  constexpr int XR = CT * TILE;                     // activation rows per k-block in LDS
  constexpr int XS = KBLK * 4 + 16;                 // LDS stride of an activation row
  constexpr bool kXL = XL > 0;                      // XL activation loads per stage, or 0
  // XP: the loading lanes split the activations, which sit in LDS as three
  // bf16 planes (hi, mid, lo; rows of 32 k, 64 bytes + 16 of padding), so
  // only the R real rows are split, once, and the operands are read as is
  static_assert(!XP || kXL, "planes need activations through LDS");
  constexpr int PS = KBLK * 2 + 16;                 // XP: LDS stride of a plane row
  constexpr int PLANE = U * XR * PS;                // XP: bytes of one plane
  constexpr int XB = !kXL ? 0 : (XP ? 3 * PLANE : U * XR * XS);  // activation stage bytes per wave
  uint8_t* stg = reinterpret_cast<uint8_t*>(red) + static_cast<size_t>(wave) * (T * TILE * RS + XB);
  uint8_t* xstg = stg + T * TILE * RS;

  // addresses: a uniform base plus this lane's 32-bit byte offset, so that
  // the per-stage step is a scalar add (the tile's rows span T * 16 * ldw * 2
  // < 2^32 bytes: ldw < 2^24 is checked on the host)
  const uint8_t* wtile = reinterpret_cast<const uint8_t*>(W + static_cast<int64_t>(n0) * ldw);
  uint32_t woffs[NI];  // this lane's rows, at its 16-byte column of the stage
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    int wr = n0 + i * RPI + lane / LPR;
    if (wr >= N) wr = N - 1;  // ragged tile: load a valid row, discard its results
    woffs[i] = static_cast<uint32_t>((wr - n0) * ldw * 2) + static_cast<uint32_t>((lane % LPR) * 16);
  }
  // Activation rows; rows >= R read row R - 1, and their (independent)
  // MFMA outputs are never stored.  Direct: the lane's own column, its two
  // 16-byte pieces at 8g and 8g + 4, loaded in the operand layout (16 rows
  // per instruction, half of each row's 128 bytes).  XL: only the R rows
  // are loaded, as whole 128-byte rows of a k-block: instruction j carries
  // the (row, k-block) pairs 8j .. 8j + 7 (pair q is row q / U, k-block
  // q % U of the stage; 8 lanes per pair), so a stage takes ceil(R U / 8)
  // instructions, and the operand layout is read back from LDS (XP: the
  // loading lanes split their four values into the bf16 planes first).
  static_assert(!kXL || (8 % U == 0 && XL <= XR * U / 8), "whole k-block pairs, at most XR rows");
  const int xu = (lane >> 3) % U;            // XL: this lane's k-block within the stage
  const int xq = (lane >> 3) / U;            // XL: its row in instruction 0
  const int xdbase = XP ? xu * XR * PS + (lane & 7) * 8    // XP: plane byte offset of row 0
                       : xu * XR * XS + (lane & 7) * 16;  // XL: LDS byte offset of row 0
  // XL: the row of this lane's pair in instruction j (rows >= R repeat row R - 1)
  auto xrow_of = [&](int j) {
    const int r = (8 / U) * j + xq;
    return r < R ? r : R - 1;
  };
  // XL: byte offsets of this lane's piece in each load from X (R * ldx * 4
  // < 2^32: ldx < 2^24 is checked on the host)
  uint32_t xoffs[kXL ? XL : 1];
#pragma unroll
  for (int j = 0; j < (kXL ? XL : 1); ++j)
    xoffs[j] = static_cast<uint32_t>(xrow_of(j)) * static_cast<uint32_t>(ldx) * 4u + static_cast<uint32_t>((lane & 7) * 16);
  const float* xrow[CT][2];
  if constexpr (!kXL) {
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = c * 16 + col;
        xrow[c][h] = X + static_cast<int64_t>(r < R ? r : R - 1) * ldx + g * 8 + h * 4;
      }
  }
  static_assert(PPW == 1 || PPW == 2, "partitions per wave");
  const int p0 = wave * PPW;
  const int kb0 = static_cast<int>((static_cast<int64_t>(p0) * nkb) / splits);
  const int kb1 = static_cast<int>((static_cast<int64_t>(p0 + PPW) * nkb) / splits);
  const int kbm = static_cast<int>((static_cast<int64_t>(p0 + 1) * nkb) / splits);  // 2nd partition
  f32x4 acc[PPW][T][CT];
#pragma unroll
  for (int q = 0; q < PPW; ++q)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int c = 0; c < CT; ++c) acc[q][t][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the stage starting at k-block kb holds blocks [kl, kl + U), kept inside
  // the wave's range: a stage issued past its end re-reads the range's last
  // blocks (cache hits) instead of the next wave's
  auto first_block = [&](int kb) { return kb + U <= kb1 ? kb : kb1 - U; };
  auto issue = [&](RunStage<T, U, CT, XL>& st, int kb) {
    // activations first: memory returns in issue order
    if constexpr (kXL) {  // ceil(R U / 8) == XL loads, none of them conditional
      const int64_t off = static_cast<int64_t>(kb + xu < kb1 ? kb + xu : kb1 - 1) * KBLK;
#pragma unroll
      for (int j = 0; j < XL; ++j)
        st.x[j] = *reinterpret_cast<const float4*>(reinterpret_cast<const uint8_t*>(X + off) + xoffs[j]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t off = static_cast<int64_t>(kb + u < kb1 ? kb + u : kb1 - 1) * KBLK;
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          st.x[(u * CT + c) * 2] = *reinterpret_cast<const float4*>(xrow[c][0] + off);
          st.x[(u * CT + c) * 2 + 1] = *reinterpret_cast<const float4*>(xrow[c][1] + off);
        }
      }
    }
    const int64_t woff = static_cast<int64_t>(first_block(kb)) * (KBLK * 2);
    const uint8_t* wstage = wtile + woff;  // uniform
#pragma unroll
    for (int i = 0; i < NI; ++i) st.w[i] = load_weights(wstage + woffs[i]);
  };
  auto compute = [&](const RunStage<T, U, CT, XL>& st, int kb) {
    const int kl = first_block(kb);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *reinterpret_cast<u32x4*>(stg + (i * RPI + lane / LPR) * RS + (lane % LPR) * 16) = st.w[i];
    if constexpr (XP) {
#pragma unroll
      for (int j = 0; j < XL; ++j) {
        uint2 hi, mid, lo;
        split3x4(st.x[j], hi, mid, lo);
        uint8_t* d = xstg + xdbase + xrow_of(j) * PS;
        *reinterpret_cast<uint2*>(d) = hi;
        *reinterpret_cast<uint2*>(d + PLANE) = mid;
        *reinterpret_cast<uint2*>(d + 2 * PLANE) = lo;
      }
    } else if constexpr (kXL) {
#pragma unroll
      for (int j = 0; j < XL; ++j)
        *reinterpret_cast<float4*>(xstg + xdbase + xrow_of(j) * XS) = st.x[j];
    }
    wave_lds_sync();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kb + u >= kb1) break;  // uniform across the wave
      const int uu = kb + u - kl;
      u32x4 a[T];
#pragma unroll
      for (int t = 0; t < T; ++t)
        a[t] = *reinterpret_cast<const u32x4*>(stg + (t * TILE + col) * RS + uu * (KBLK * 2) + g * 16);
      auto accumulate = [&](f32x4 (&ac)[T][CT]) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          u32x4 hi, mid, lo;
          if constexpr (XP) {
            const int r = c * TILE + col < R ? c * TILE + col : R - 1;  // rows >= R: never stored
            const uint8_t* xa = xstg + (u * XR + r) * PS + g * 16;
            hi = *reinterpret_cast<const u32x4*>(xa);
            mid = *reinterpret_cast<const u32x4*>(xa + PLANE);
            lo = *reinterpret_cast<const u32x4*>(xa + 2 * PLANE);
          } else {
            float4 x0, x1;
            if constexpr (kXL) {
              const int r = c * TILE + col < R ? c * TILE + col : R - 1;  // rows >= R: never stored
              const uint8_t* xa = xstg + (u * XR + r) * XS + g * 32;
              x0 = *reinterpret_cast<const float4*>(xa);
              x1 = *reinterpret_cast<const float4*>(xa + 16);
            } else {
              x0 = st.x[(u * CT + c) * 2];
              x1 = st.x[(u * CT + c) * 2 + 1];
            }
            const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            split3(xv, hi, mid, lo);
          }
#pragma unroll
          for (int t = 0; t < T; ++t) {
            ac[t][c] = mfma(a[t], hi, ac[t][c]);
            ac[t][c] = mfma(a[t], mid, ac[t][c]);
            ac[t][c] = mfma(a[t], lo, ac[t][c]);
          }
        }
      };
      if (PPW == 1 || kb + u < kbm) accumulate(acc[0]);  // uniform across the wave
      else accumulate(acc[PPW - 1]);
    }
    wave_lds_sync();  // every lane has read the stage before the next one is written
  };
  if (kb0 < kb1) {
    RunStage<T, U, CT, XL> sa, sb;
    issue(sa, kb0);
    for (int kb = kb0; kb < kb1; kb += 2 * U) {
      issue(sb, kb + U);
      compute(sa, kb);
      issue(sa, kb + 2 * U);
      compute(sb, kb + U);
    }
  }
  __syncthreads();  // the stage buffers become the reduction buffer

  // Partition sums meet in LDS and are added in partition order.
#pragma unroll
  for (int q = 0; q < PPW; ++q)
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          red[((((p0 + q) * T + t) * CT + c) * 4 + e) * 64 + lane] = acc[q][t][c][e];
  __syncthreads();
  const int per_wave = T * CT * 256;
  for (int idx = threadIdx.x; idx < per_wave; idx += blockDim.x) {
    float s = red[idx];
    for (int w = 1; w < splits; ++w) s += red[w * per_wave + idx];
    const int l = idx & 63;
    const int e = (idx >> 6) & 3;
    const int c = (idx >> 8) % CT;
    const int t = (idx >> 8) / CT;
    const int n = n0 + t * TILE + 4 * (l >> 4) + e;
    const int r = c * 16 + (l & 15);
    if (n < N && r < R) Y[static_cast<int64_t>(r) * ldy + n] = s;
  }
}

// Activations of one pipeline stage in the MFMA B-operand layout, split into
// three bf16 planes: [U k-blocks][hi, mid, lo][CT column tiles][64 lanes].
template <int U, int CT>
struct XTile {
  u32x4 v[U][3][CT][64];
};

// Shared-activation kernel.  Workgroup = P wavefronts; wave p owns the T
// 16-row tiles starting at row (blockIdx.x * P + p) * 16 * T.  SPLITK: the
// workgroup takes partition blockIdx.y and writes its partial sums to
// parts[(s * R + r) * ldp + n]; otherwise each wave walks all partitions and
// writes Y.  Stage s + 1 (weights in registers, activations split into the
// other LDS buffer) is loaded while stage s is computed.
template <int T, int U, int CT, int P, bool SPLITK>
__global__ void __launch_bounds__(64 * P)
gemv_shared_kernel(const uint16_t* __restrict__ W, int64_t ldw, int N, int K,
                   const float* __restrict__ X, int64_t ldx, int R, float* __restrict__ Y,
                   int64_t ldy, float* __restrict__ parts, int64_t ldp, int nkb, int splits) {
  __shared__ XTile<U, CT> xs[2];
  constexpr int IMG = U * CT;             // activation images (one k-block, one column tile) per stage
  constexpr int IPW = (IMG + P - 1) / P;  // images each wave loads and splits
  const int lane = threadIdx.x & 63;
  const int p = vs::wave_index();
  const int g = lane >> 4;
  const int col = lane & 15;
  const int n0 = (blockIdx.x * P + p) * TILE * T;
  int kb0 = 0, kb1 = nkb;
  if (SPLITK) {
    kb0 = static_cast<int>((static_cast<int64_t>(blockIdx.y) * nkb) / splits);
    kb1 = static_cast<int>((static_cast<int64_t>(blockIdx.y + 1) * nkb) / splits);
  }

  const uint16_t* wrow[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    int wr = n0 + t * TILE + col;
    if (wr >= N) wr = N - 1;  // ragged tile: load a valid row, discard its results
    wrow[t] = W + static_cast<int64_t>(wr) * ldw + g * 8;
  }
  f32x4 acc[T][CT], y[T][CT];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      y[t][c] = acc[t][c];
    }

  auto load_w = [&](u32x4 (&w)[U][T], int kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = kb + u < kb1 && (kb + u) * KBLK + g * 8 < K;  // K % 8 == 0
      const int64_t off = static_cast<int64_t>(kb + u) * KBLK;
#pragma unroll
      for (int t = 0; t < T; ++t)
        // plain loads: with the non-temporal hint this kernel ran 10% slower
        w[u][t] = ok ? *reinterpret_cast<const u32x4*>(wrow[t] + off) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto load_x = [&](float (&x)[IPW][8], int kb) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int img = p + i * P;
      const int u = img / CT, c = img % CT;
      const int r = c * 16 + col;
      const int k = (kb + u) * KBLK + g * 8;
      if (img < IMG && kb + u < kb1 && k < K && r < R) {
        const float* src = X + static_cast<int64_t>(r) * ldx + k;
        const float4 a = *reinterpret_cast<const float4*>(src);
        const float4 b = *reinterpret_cast<const float4*>(src + 4);
        x[i][0] = a.x; x[i][1] = a.y; x[i][2] = a.z; x[i][3] = a.w;
        x[i][4] = b.x; x[i][5] = b.y; x[i][6] = b.z; x[i][7] = b.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
      }
    }
  };
  auto store_x = [&](const float (&x)[IPW][8], int buf) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int img = p + i * P;
      if (img < IMG) {
        const int u = img / CT, c = img % CT;
        u32x4 hi, mid, lo;
        split3(x[i], hi, mid, lo);
        xs[buf].v[u][0][c][lane] = hi;
        xs[buf].v[u][1][c][lane] = mid;
        xs[buf].v[u][2][c][lane] = lo;
      }
    }
  };
  // all-K mode: partition `part` ends at k-block `bound`; its sum is added
  // into y (left to right) and the accumulator restarts from zero
  int part = 0;
  int bound = static_cast<int>(static_cast<int64_t>(nkb) / splits);
  auto flush_to = [&](int kb) {
    while (part < splits && bound <= kb) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          y[t][c] = part == 0 ? acc[t][c] : y[t][c] + acc[t][c];
          acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      ++part;
      bound = static_cast<int>((static_cast<int64_t>(part + 1) * nkb) / splits);
    }
  };

  u32x4 w[U][T];
  float x[IPW][8];
  load_w(w, kb0);
  load_x(x, kb0);
  store_x(x, 0);
  __syncthreads();
  if (!SPLITK) flush_to(kb0);
  int buf = 0;
  for (int kb = kb0; kb < kb1; kb += U) {  // uniform over the workgroup
    const bool more = kb + U < kb1;
    u32x4 wn[U][T];
    if (more) {
      load_x(x, kb + U);
      load_w(wn, kb + U);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kb + u >= kb1) break;
      if (!SPLITK && kb + u == bound) flush_to(kb + u);
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const u32x4 hi = xs[buf].v[u][0][c][lane];
        const u32x4 mid = xs[buf].v[u][1][c][lane];
        const u32x4 lo = xs[buf].v[u][2][c][lane];
#pragma unroll
        for (int t = 0; t < T; ++t) {
          acc[t][c] = mfma(w[u][t], hi, acc[t][c]);
          acc[t][c] = mfma(w[u][t], mid, acc[t][c]);
          acc[t][c] = mfma(w[u][t], lo, acc[t][c]);
        }
      }
    }
    if (more) {
      store_x(x, buf ^ 1);  // the other buffer was last read before the previous barrier
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < T; ++t) w[u][t] = wn[u][t];
    }
    __syncthreads();
    buf ^= 1;
  }

  // MFMA 16x16 output layout: lane l, element e holds weight row 4*(l/16)+e
  // of the tile and activation row l%16 of the column tile.
  if (SPLITK) {
    const int64_t pbase = static_cast<int64_t>(blockIdx.y) * R;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int r = c * 16 + col;
        const int n = n0 + t * TILE + 4 * g;
        if (r >= R || n >= N) continue;
        float* dst = parts + (pbase + r) * ldp + n;
        if (n + 3 < N) {
          *reinterpret_cast<f32x4*>(dst) = acc[t][c];  // ldp % 4 == 0, n % 4 == 0
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) dst[e] = acc[t][c][e];
        }
      }
  } else {
    flush_to(kb1);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int r = c * 16 + col;
        const int n = n0 + t * TILE + 4 * g;
        if (r >= R) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N) Y[static_cast<int64_t>(r) * ldy + n + e] = y[t][c][e];
      }
  }
}

// Staged split-K kernel: the shared kernel's activation planes (each
// k-block's activations split once per workgroup into LDS) with the staged
// kernel's weight path (row runs of 8 rows x 128 bytes per load,
// non-temporal, no per-lane guards, restaged through the wave's own LDS
// region into the operand layout).  Workgroup = P wavefronts along N, wave p
// owning T 16-row tiles, over partition blockIdx.y, whose sums go to
// parts[(s * R + r) * ldp + n] for reduce_partials_kernel.  Every wave loads
// one activation image per stage (images past the stage's count are loaded
// but not stored, so that no load is conditional).  Requires K % 32 == 0
// and at least U k-blocks per partition.
template <int T, int CT, int P>
__global__ void __launch_bounds__(64 * P)
gemv_staged_split_kernel(const uint16_t* __restrict__ W, int64_t ldw, int N, int K,
                         const float* __restrict__ X, int64_t ldx, int R,
                         float* __restrict__ parts, int64_t ldp, int nkb, int splits) {
  constexpr int U = 2;                    // k-blocks per stage
  constexpr int RB = U * KBLK * 2;        // bytes of one weight row per stage
  constexpr int RS = RB + 16;             // LDS row stride
  constexpr int LPR = RB / 16;            // lanes per row in one load
  constexpr int RPI = 64 / LPR;           // rows per load instruction
  constexpr int NI = T * TILE / RPI;      // weight loads per stage
  constexpr int IMG = U * CT;             // activation images per stage
  constexpr int IPW = (IMG + P - 1) / P;  // images each wave loads
  static_assert(64 % LPR == 0 && (T * TILE) % RPI == 0, "stage shape");
  __shared__ XTile<U, CT> xs[2];
  extern __shared__ float wst[];          // [P][T * TILE * RS bytes]
  const int lane = threadIdx.x & 63;
  const int p = vs::wave_index();
  const int g = lane >> 4;
  const int col = lane & 15;
  const int n0 = (blockIdx.x * P + p) * TILE * T;
  const int kb0 = static_cast<int>((static_cast<int64_t>(blockIdx.y) * nkb) / splits);
  const int kb1 = static_cast<int>((static_cast<int64_t>(blockIdx.y + 1) * nkb) / splits);
  uint8_t* stg = reinterpret_cast<uint8_t*>(wst) + static_cast<size_t>(p) * (T * TILE * RS);

  const uint8_t* wsrc[NI];  // this lane's rows, at its 16-byte column of the stage
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    int wr = n0 + i * RPI + lane / LPR;
    if (wr >= N) wr = N - 1;  // ragged tile: load a valid row, discard its results
    wsrc[i] = reinterpret_cast<const uint8_t*>(W + static_cast<int64_t>(wr) * ldw) + (lane % LPR) * 16;
  }
  // this wave's activation images: (k-block u, column tile c) = img / CT,
  // img % CT; the lane's row (rows >= R repeat row R - 1, never stored) and
  // its 8 values at k = 32 (kb + u) + 8 g
  const float* xsrc[IPW];
  int ximg[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    ximg[i] = p + i * P;
    const int img = ximg[i] % IMG;
    const int c = img % CT;
    const int r = c * TILE + col < R ? c * TILE + col : R - 1;
    xsrc[i] = X + static_cast<int64_t>(r) * ldx + g * 8;
  }

  f32x4 acc[T][CT];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // a stage starting at k-block kb holds blocks [kl, kl + U), kept inside the
  // range: a stage issued past the end re-reads the range's last blocks
  auto first_block = [&](int kb) { return kb + U <= kb1 ? kb : kb1 - U; };
  auto issue = [&](float (&x)[IPW][8], u32x4 (&w)[NI], int kb) {
    // activations first: memory returns in issue order
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int u = (ximg[i] % IMG) / CT;
      const int64_t off = static_cast<int64_t>(kb + u < kb1 ? kb + u : kb1 - 1) * KBLK;
      const float4 a = *reinterpret_cast<const float4*>(xsrc[i] + off);
      const float4 b = *reinterpret_cast<const float4*>(xsrc[i] + off + 4);
      x[i][0] = a.x; x[i][1] = a.y; x[i][2] = a.z; x[i][3] = a.w;
      x[i][4] = b.x; x[i][5] = b.y; x[i][6] = b.z; x[i][7] = b.w;
    }
    const int64_t woff = static_cast<int64_t>(first_block(kb)) * (KBLK * 2);
#pragma unroll
    for (int i = 0; i < NI; ++i) w[i] = load_weights(wsrc[i] + woff);
  };
  auto store_x = [&](const float (&x)[IPW][8], int buf) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      if (ximg[i] < IMG) {  // uniform across the wave
        const int u = ximg[i] / CT, c = ximg[i] % CT;
        u32x4 hi, mid, lo;
        split3(x[i], hi, mid, lo);
        xs[buf].v[u][0][c][lane] = hi;
        xs[buf].v[u][1][c][lane] = mid;
        xs[buf].v[u][2][c][lane] = lo;
      }
    }
  };
  // one stage: weights w (k-blocks from kb) against activation buffer buf;
  // the next stage's loads (xn, wn) are issued first
  float x[IPW][8];
  auto stage = [&](const u32x4 (&w)[NI], u32x4 (&wn)[NI], int kb, int buf) {
    issue(x, wn, kb + U);
    const int kl = first_block(kb);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *reinterpret_cast<u32x4*>(stg + (i * RPI + lane / LPR) * RS + (lane % LPR) * 16) = w[i];
    wave_lds_sync();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kb + u >= kb1) break;  // uniform across the workgroup
      const int uu = kb + u - kl;
      u32x4 a[T];
#pragma unroll
      for (int t = 0; t < T; ++t)
        a[t] = *reinterpret_cast<const u32x4*>(stg + (t * TILE + col) * RS + uu * (KBLK * 2) + g * 16);
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const u32x4 hi = xs[buf].v[u][0][c][lane];
        const u32x4 mid = xs[buf].v[u][1][c][lane];
        const u32x4 lo = xs[buf].v[u][2][c][lane];
#pragma unroll
        for (int t = 0; t < T; ++t) {
          acc[t][c] = mfma(a[t], hi, acc[t][c]);
          acc[t][c] = mfma(a[t], mid, acc[t][c]);
          acc[t][c] = mfma(a[t], lo, acc[t][c]);
        }
      }
    }
    wave_lds_sync();  // every lane has read the weights before the next stage's are written
    store_x(x, buf ^ 1);  // that buffer was last read before the previous barrier
    __syncthreads();
  };

  u32x4 wa[NI], wb[NI];
  issue(x, wa, kb0);
  store_x(x, 0);
  __syncthreads();
  for (int kb = kb0; kb < kb1; kb += 2 * U) {  // uniform over the workgroup
    stage(wa, wb, kb, 0);
    if (kb + U >= kb1) break;
    stage(wb, wa, kb + U, 1);
  }

  // MFMA 16x16 output layout: lane l, element e holds weight row 4*(l/16)+e
  // of the tile and activation row l%16 of the column tile.
  const int64_t pbase = static_cast<int64_t>(blockIdx.y) * R;
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int r = c * 16 + col;
      const int n = n0 + t * TILE + 4 * g;
      if (r >= R || n >= N) continue;
      float* dst = parts + (pbase + r) * ldp + n;
      if (n + 3 < N) {
        *reinterpret_cast<f32x4*>(dst) = acc[t][c];  // ldp % 4 == 0, n % 4 == 0
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < N) dst[e] = acc[t][c][e];
      }
    }
}

// Y[r][n..n+3] = the partition sums of parts added left to right.  All
// partition loads are issued before the first add (the add order is fixed,
// the load order is not), so the kernel costs one memory round trip.
//
// The split-K kernels write the partial sums of row block g (rows_g rows)
// from workgroups g + ngroups * s of a (ngroups, splits) grid, all on XCD
// g % 8 when ngroups % 8 == 0 (workgroups are dealt to the eight XCDs round
// robin in launch order), and a line written by one kernel is still in that
// XCD's L2 for the next (read back 2.2x faster than from another XCD on
// MI355X).  So workgroup id = (g / 8 * RS + slice) * 8 + g % 8 adds block
// g's sums for rows [slice * per, slice * per + per), per = 256 / (rows_g /
// 4), on the XCD that wrote them: 7-28 us less per 36-layer pass where the
// split-K kernel runs.  Any other mapping gives the same bits.
constexpr int MAX_SPLITS = 16;

__global__ void __launch_bounds__(256)
reduce_partials_kernel(const float* __restrict__ parts, int64_t ldp, int splits, int R, int N,
                       float* __restrict__ Y, int64_t ldy, int ngroups, int rows_g, int RS) {
  const int id = static_cast<int>(blockIdx.x);
  const int j = id >> 3;
  const int g = (j / RS) * 8 + (id & 7);
  if (g >= ngroups) return;
  const int quads = rows_g / 4;   // 16 or 32
  const int per = 256 / quads;    // rows per workgroup
  const int r = (j % RS) * per + static_cast<int>(threadIdx.x) / quads;
  const int n = g * rows_g + (static_cast<int>(threadIdx.x) % quads) * 4;
  if (r >= R || n >= N) return;
  f32x4 v[MAX_SPLITS];
#pragma unroll
  for (int q = 0; q < MAX_SPLITS; ++q)
    if (q < splits)  // ldp % 4 == 0 and n % 4 == 0: 16-byte aligned, inside the row's ldp
      v[q] = *reinterpret_cast<const f32x4*>(parts + (static_cast<int64_t>(q) * R + r) * ldp + n);
  f32x4 s = v[0];
#pragma unroll
  for (int q = 1; q < MAX_SPLITS; ++q)
    if (q < splits) s += v[q];
  float* dst = Y + static_cast<int64_t>(r) * ldy + n;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (n + e < N) dst[e] = s[e];
}

// Launches reduce_partials_kernel for a split-K grid of row blocks of rows_g
// (64 or 128) rows.
int launch_reduce(const float* parts, int64_t ldp, int splits, int R, int N, float* Y, int64_t ldy,
                  int rows_g, hipStream_t stream) {
  const int ngroups = (N + rows_g - 1) / rows_g;
  const int per = 256 / (rows_g / 4);
  const int RS = (R + per - 1) / per;
  reduce_partials_kernel<<<dim3(static_cast<unsigned>(((ngroups + 7) / 8) * 8 * RS)), dim3(256), 0, stream>>>(
      parts, ldp, splits, R, N, Y, ldy, ngroups, rows_g, RS);
  return vs::check_launch();
}

// K partitions (the k-split): a function of N and K alone, so that the
// summation order of a row does not change with R.
//  * Wide matrices (N >= 16384: enough row tiles to fill the chip) take few,
//    long partitions: the fewest with at most 32 k-blocks each whose length
//    is a whole number of the staged kernel's 4-k-block pipeline
//    iterations (a ragged partition costs a partial iteration in every wave;
//    on 151936 x 2560, 3 ragged partitions ran at 0.61 of peak, 4 or 5 whole
//    ones at 0.78-0.80);
//  * narrower ones split K further for parallelism: 8 partitions, or 16 for
//    long rows (the staged row-block kernel then walks two partitions per
//    wave and keeps its wave count, the split-K kernel gets 16 workgroups
//    per row block).
// Chosen by sweeps of 15 matrices of three model sizes on MI355X.
int splits_for(int N, int K) {
  const int nkb = (K + KBLK - 1) / KBLK;
  if (N >= 16384) {
    const int lo = (nkb + 31) / 32 < 1 ? 1 : (nkb + 31) / 32;
    for (int s = lo; s <= MAX_SPLITS; ++s)
      if (nkb % s == 0 && (nkb / s) % 4 == 0 && (s <= 8 || s % 2 == 0)) return s;
    return lo < MAX_SPLITS ? lo : MAX_SPLITS;
  }
  if (nkb >= 256) return 16;  // long rows (4096 x 12288): more, shorter partitions
  const int s = (nkb + 15) / 16 < 8 ? (nkb + 15) / 16 : 8;
  return s < 1 ? 1 : s;  // <= MAX_SPLITS
}

// Whether the staged row-block kernel can take (N, K): whole k-blocks, at
// least two stages per partition, and an even partition count above 8.
bool staged_fits(int N, int K) {
  const int nkb = (K + KBLK - 1) / KBLK;
  const int splits = splits_for(N, K);
  return K % KBLK == 0 && nkb / splits >= 2 && (splits <= 8 || splits % 2 == 0);
}

// The share of the chip's workgroup slots that G workgroups use when each
// CU runs one at a time: G over the slots of all the rounds they take.
constexpr double CUS = 256.0;
double fill(double G) { return G / (CUS * std::ceil(G / CUS)); }

// Whether the staged split-K kernel (and its partition-sum launch) is
// modelled faster than the staged row-block kernel at R <= 16 rows.  Each
// kernel's time is the bytes it moves over an effective bandwidth scaled by
// how well its grid fills the CUs:
//   row-block: weights + the activations that each row tile re-reads,
//   split-K:   weights + each workgroup's activation slice + the partial
//              sums written and read back, plus the dependent launch.
// Activation re-reads are mostly L2 hits and count 0.3 of an HBM byte.  The
// constants (7 TB/s, 5 us, 0.3) are fitted to row-block and split-K timings
// of 13 matrices of three model sizes at R = 1..16 on MI355X; the tile
// heights are the ones the dispatch below launches.
bool split_k_pays(int N, int K, int R) {
  constexpr double BW = 7.0e12, LAUNCH_S = 5e-6, ACT = 0.3;
  const int nkb = (K + KBLK - 1) / KBLK;
  const int s = splits_for(N, K);
  const int t_rb = N < 6144 ? 1 : 2;                       // row tiles per row-block wave
  const int t_sk = (nkb >= 256 || N >= 16384) ? 2 : 1;     // per split-K wave (4 waves)
  const double g_rb = std::ceil(N / (16.0 * t_rb));
  const double g_sk = std::ceil(N / (64.0 * t_sk)) * s;
  const double w = 2.0 * N * K;
  const double t_row = (w + ACT * g_rb * R * K * 4.0) / (BW * fill(g_rb));
  const double t_split = (w + ACT * g_sk * R * (static_cast<double>(K) / s) * 4.0 + 8.0 * R * N * s) /
                             (BW * fill(g_sk)) + LAUNCH_S;
  return t_split < t_row;
}

// Which kernel runs for (N, K, R).  The row-block kernels re-read the
// activations once per row tile, so their time grows with R; the split-K
// kernels share each activation tile among a workgroup's waves and stay
// nearly flat in R, from a higher base (a dependent partition-sum launch),
// and their grid (row blocks x partitions) fills the chip where the
// row-block grid leaves a part of a round idle.  Matrices under 48 MB and
// the LM head (whose partial sums would cost more than the shared
// activations save) always take the row-block kernel.  Otherwise the
// split-K kernel runs above 16 rows (where the row-block kernel needs a
// second activation column tile), from 9 rows for long rows, and wherever
// split_k_pays models it faster.  Where the staged kernels cannot run
// (K % 32 != 0), matrices of >= 48 MB take the older shared kernels from 9
// rows (long rows) or above 16 rows (all-K for very wide ones).
enum class Kind { kRowBlock, kSharedAllK, kSharedSplitK, kStagedSplitK };

Kind kind_for(int N, int K, int R) {
  const bool big = 2.0 * N * K >= 48e6;
  const bool long_rows = (K + KBLK - 1) / KBLK >= 256;
  if (staged_fits(N, K)) {
    if (!big || N >= 65536) return Kind::kRowBlock;
    if (R > 16 || (long_rows && R >= 9) || split_k_pays(N, K, R)) return Kind::kStagedSplitK;
    return Kind::kRowBlock;
  }
  if (R <= 8) return Kind::kRowBlock;
  if (N < 65536 && big && long_rows) return Kind::kSharedSplitK;
  if (R <= 16 || !big) return Kind::kRowBlock;
  return N >= 65536 ? Kind::kSharedAllK : Kind::kSharedSplitK;
}

int64_t parts_ld(int N) { return (static_cast<int64_t>(N) + 3) & ~int64_t{3}; }

size_t split_workspace_bytes(int N, int K, int R) {
  return static_cast<size_t>(splits_for(N, K)) * R * parts_ld(N) * sizeof(float);
}

}  // namespace

extern "C" size_t verify_gemv_rows_workspace_bytes(int N, int K, int R) {
  if (N < 1 || K < 1 || R < 1 || R > VS_MAX_ROWS) return 0;
  const Kind kind = kind_for(N, K, R);
  return kind == Kind::kSharedSplitK || kind == Kind::kStagedSplitK ? split_workspace_bytes(N, K, R) : 0;
}

extern "C" int verify_gemv_rows(const uint16_t* W, int64_t ldw, int N, int K, const float* X,
                                int64_t ldx, int R, float* Y, int64_t ldy, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (!W || !X || !Y) return VS_ERR_NULL;
  if (N < 1 || K < 1 || R < 1 || R > VS_MAX_ROWS) return VS_ERR_SHAPE;
  if (K % 8 != 0 || ldw < K || ldx < K || ldy < N) return VS_ERR_SHAPE;
  if (ldw % 8 != 0 || ldx % 4 != 0 || !vs::aligned16(W) || !vs::aligned16(X)) return VS_ERR_ALIGN;
  if (static_cast<int64_t>(N) > (int64_t{1} << 31) - 1024) return VS_ERR_SHAPE;
  if (ldw >= (int64_t{1} << 24) || ldx >= (int64_t{1} << 24)) return VS_ERR_SHAPE;  // 32-bit tile offsets

  const int nkb = (K + KBLK - 1) / KBLK;
  const int splits = splits_for(N, K);
  Kind kind = kind_for(N, K, R);
  // without a (large enough, aligned) workspace the row-block kernel runs:
  // same summation order, same bits
  if ((kind == Kind::kSharedSplitK || kind == Kind::kStagedSplitK) &&
      (!workspace || workspace_bytes < split_workspace_bytes(N, K, R) || !vs::aligned16(workspace)))
    kind = Kind::kRowBlock;

  if (kind == Kind::kStagedSplitK) {
    float* parts = static_cast<float*>(workspace);
    const int64_t ldp = parts_ld(N);
    auto launch = [&](auto kernel, int T, int P) {
      const dim3 grid((N + TILE * T * P - 1) / (TILE * T * P), splits);
      const size_t shm = static_cast<size_t>(P) * T * TILE * (2 * KBLK * 2 + 16);
      kernel<<<grid, dim3(64 * P), shm, stream>>>(W, ldw, N, K, X, ldx, R, parts, ldp, nkb, splits);
    };
    // 32-row tiles per wave for long rows and wide matrices, 16 for the
    // q|k|v-sized ones (chosen by sweep)
    const bool tall = (K + KBLK - 1) / KBLK >= 256 || N >= 16384;
    if (tall) {
      if (R > 16) launch(gemv_staged_split_kernel<2, 2, 4>, 2, 4);
      else launch(gemv_staged_split_kernel<2, 1, 4>, 2, 4);
    } else {
      if (R > 16) launch(gemv_staged_split_kernel<1, 2, 4>, 1, 4);
      else launch(gemv_staged_split_kernel<1, 1, 4>, 1, 4);
    }
    int st = vs::check_launch();
    if (st != VS_OK) return st;
    return launch_reduce(parts, ldp, splits, R, N, Y, ldy, TILE * (tall ? 2 : 1) * 4, stream);
  }
  if (kind == Kind::kSharedAllK) {
    auto launch = [&](auto kernel, int T, int P) {
      const dim3 grid((N + TILE * T * P - 1) / (TILE * T * P));
      kernel<<<grid, dim3(64 * P), 0, stream>>>(W, ldw, N, K, X, ldx, R, Y, ldy, nullptr, 0, nkb,
                                                splits);
    };
    launch(gemv_shared_kernel<1, 2, 2, 8, false>, 1, 8);  // R > 16: two column tiles
    return vs::check_launch();
  }
  if (kind == Kind::kSharedSplitK) {
    float* parts = static_cast<float*>(workspace);
    const int64_t ldp = parts_ld(N);
    auto launch = [&](auto kernel, int T, int P) {
      const dim3 grid((N + TILE * T * P - 1) / (TILE * T * P), splits);
      kernel<<<grid, dim3(64 * P), 0, stream>>>(W, ldw, N, K, X, ldx, R, Y, ldy, parts, ldp, nkb,
                                                splits);
    };
    if (R > 16) {  // two activation column tiles
      if (N >= 16384) launch(gemv_shared_kernel<1, 2, 2, 8, true>, 1, 8);
      else launch(gemv_shared_kernel<1, 2, 2, 4, true>, 1, 4);
    } else {
      if (N >= 16384) launch(gemv_shared_kernel<1, 2, 1, 8, true>, 1, 8);
      else launch(gemv_shared_kernel<1, 2, 1, 4, true>, 1, 4);
    }
    int st = vs::check_launch();
    if (st != VS_OK) return st;
    return launch_reduce(parts, ldp, splits, R, N, Y, ldy, TILE * (N >= 16384 ? 8 : 4), stream);
  }

  const dim3 block(64 * splits);
  // Staged row-block kernel wherever its conditions hold.
  constexpr int STAGE_U = 2;
  static_assert(STAGE_U == 2, "staged_fits assumes two k-blocks per stage");
  if (staged_fits(N, K)) {
    const int ppw = splits > 8 ? 2 : 1;  // partitions per wave: at most 8 waves
    const int waves = splits / ppw;
    auto launch_staged = [&](auto kernel, int T, int CT, bool xl, bool xp = false) {
      const dim3 grid((N + TILE * T - 1) / (TILE * T));
      size_t shm = static_cast<size_t>(splits) * T * CT * 256 * sizeof(float);
      const size_t xbytes = !xl ? 0
                            : xp ? 3 * STAGE_U * CT * TILE * (KBLK * 2 + 16)
                                 : STAGE_U * CT * TILE * (KBLK * 4 + 16);
      const size_t stage = static_cast<size_t>(waves) * (T * TILE * (STAGE_U * KBLK * 2 + 16) + xbytes);
      if (stage > shm) shm = stage;
      kernel<<<grid, dim3(64 * waves), shm, stream>>>(W, ldw, N, K, X, ldx, R, Y, ldy, nkb, splits);
    };
    // T row tiles and CT column tiles, activations through LDS with
    // ceil(R U / 8) loads per stage (a compile-time count); xp: split by the
    // loading lanes into bf16 planes (4-7% faster on the layer shapes at
    // R <= 8, where the split otherwise repeats for all 16 operand rows;
    // 7-9% slower for the LM head's 64-row tiles above 16 rows, whose larger
    // LDS share leaves one workgroup per CU)
    const int nx = (R * STAGE_U + 7) / 8;
    auto staged = [&](auto t_c, auto ct_c, auto xp_c) {
      constexpr int T = decltype(t_c)::value, CT = decltype(ct_c)::value;
      constexpr bool XP = decltype(xp_c)::value;
      auto go = [&](auto xl_c) {
        constexpr int XL = decltype(xl_c)::value;
        if (ppw == 2) launch_staged(gemv_rows_staged_kernel<T, STAGE_U, CT, 512, 2, XL, XP>, T, CT, true, XP);
        else launch_staged(gemv_rows_staged_kernel<T, STAGE_U, CT, 512, 1, XL, XP>, T, CT, true, XP);
      };
      if constexpr (CT == 1) {
        if (nx == 1) go(std::integral_constant<int, 1>{});
        else if (nx == 2) go(std::integral_constant<int, 2>{});
        else if (nx == 3) go(std::integral_constant<int, 3>{});
        else go(std::integral_constant<int, 4>{});
      } else {  // R > 16
        if (nx == 5) go(std::integral_constant<int, 5>{});
        else go(std::integral_constant<int, 6>{});
      }
    };
    using Planes = std::true_type;
    using One = std::integral_constant<int, 1>;
    using Two = std::integral_constant<int, 2>;
    using Four = std::integral_constant<int, 4>;
    if (N < 6144) {  // 16-row tiles
      if (R <= 16) staged(One{}, One{}, Planes{});
      else staged(One{}, Two{}, Planes{});
    } else if (R > 16 && N < 16384) {  // q|k|v-sized: 32-row tiles, two column tiles
      staged(Two{}, Two{}, Planes{});
    } else if (R > 16) {  // gate|up and the LM head: 64-row tiles, two column tiles
      staged(Four{}, Two{}, std::false_type{});
    } else if (N >= 65536 && R > 8) {
      // 128-row tiles, activations loaded in the operand layout (through LDS
      // they were 2-3% slower here)
      launch_staged(gemv_rows_staged_kernel<8, STAGE_U, 1, 512, 1, 0>, 8, 1, false);
    } else {  // 32-row tiles, R <= 16
      staged(Two{}, One{}, Planes{});
    }
    return vs::check_launch();
  }
  // Row-block tile shape by matrix shape and R (it never changes a row's
  // summation order): taller matrices take more row tiles per wave, which
  // divides the activation traffic and the splitting work per weight;
  // "activations first" issues a stage's activation loads ahead of its
  // weights so that their split overlaps the weight latency.  Chosen by a
  // sweep on MI355X.
  auto launch = [&](auto kernel, int T, int CT) {
    const dim3 grid((N + TILE * T - 1) / (TILE * T));
    const size_t shm = static_cast<size_t>(splits) * T * CT * 256 * sizeof(float);
    kernel<<<grid, block, shm, stream>>>(W, ldw, N, K, X, ldx, R, Y, ldy, nkb, splits);
  };
  if (R <= 16) {
    if (N >= 65536 && R > 8) launch(gemv_rows_kernel<4, 1, 1, true>, 4, 1);
    else if (N >= 65536) launch(gemv_rows_kernel<2, 4, 1, true>, 2, 1);
    else if (N >= 16384 && R > 8) launch(gemv_rows_kernel<2, 2, 1, false>, 2, 1);
    else if (N >= 6144) launch(gemv_rows_kernel<2, 2, 1, true>, 2, 1);
    else launch(gemv_rows_kernel<1, 4, 1, true>, 1, 1);
  } else {
    if (N >= 65536) launch(gemv_rows_kernel<4, 1, 2, true>, 4, 2);
    else if (N >= 6144) launch(gemv_rows_kernel<2, 2, 2, true>, 2, 2);
    else launch(gemv_rows_kernel<1, 2, 2, true>, 1, 2);
  }
  return vs::check_launch();
}
