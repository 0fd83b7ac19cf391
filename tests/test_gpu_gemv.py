"""GPU parity of verify_gemv_rows against the fp64 oracle.

Tolerance: |y_gpu - y_ref| <= 1e-4 * sum_k |w*x| per element.  Row identity:
row r of an R-row call equals the 1-row call on X[r] bit for bit ("the
multi-row projections sum in exactly the single-row decode order", section
02 of "Speculative decoding on RDNA").
"""

import numpy as np
import pytest
import torch

import verify_sampling_amd as vs
from gpu_common import dev, host
from oracle.gemv import gemv_rows
from synth import (FAMILY_SHAPES, LAYER_SHAPES, LAYER_SHAPES_FUSED, LM_HEAD_SHAPE, gemv_case,
                   torch_bf16_weights)

pytestmark = pytest.mark.gpu
TOL = 1e-4


def check(y, w_bits, x, rows=None):
    ref, s = gemv_rows(w_bits, x, rows=rows)
    yy = y if rows is None else y[:, rows]
    err = np.abs(yy.astype(np.float64) - ref)
    bad = err > TOL * s
    assert not bad.any(), f"{bad.sum()} elements out of tolerance, worst {err.max()}"
    return float((err / np.maximum(s, 1e-300)).max())


@pytest.mark.parametrize("N,K,R", [(1024, 1024, 1), (1024, 1024, 2), (1024, 1024, 4),
                                   (1024, 1024, 8), (1000, 1000, 1), (1000, 1000, 3),
                                   (1000, 1000, 16), (1000, 1000, 17), (1000, 1000, 24),
                                   (1, 8, 1), (17, 40, 24), (33, 4104, 5), (5, 12296, 24)])
def test_parity_small_and_ragged(N, K, R):
    w, x = gemv_case(1000 + N + K + R, N, K, R)
    y = host(vs.verify_gemv_rows(dev(w), dev(x)))
    check(y, w, x)


@pytest.mark.parametrize("N,K", [(1024, 1024), (1000, 1000), (4096, 4096), (1024, 12288)])
def test_rows_bit_identical_to_single_row(N, K):
    w, x = gemv_case(2000 + N + K, N, K, 24)
    W, X = dev(w), dev(x)
    single = np.stack([host(vs.verify_gemv_rows(W, X[r:r + 1]))[0] for r in range(24)])
    for R in range(1, 25):
        y = host(vs.verify_gemv_rows(W, X[:R].contiguous()))
        assert np.array_equal(y.view(np.uint32), single[:R].view(np.uint32)), f"R={R}"


def test_layer_projections_r4_and_r1():
    """One 8B-class layer's seven projections at R = 4, checked in full, plus R = 1."""
    for i, (name, (N, K)) in enumerate(LAYER_SHAPES.items()):
        w, x = gemv_case(1200 + i, N, K, 4)
        W, X = dev(w), dev(x)
        y4 = host(vs.verify_gemv_rows(W, X))
        check(y4, w, x)
        for r in range(4):
            y1 = host(vs.verify_gemv_rows(W, X[r:r + 1]))
            assert np.array_equal(y1[0].view(np.uint32), y4[r].view(np.uint32)), (name, r)


def sampled_rows(N, n, seed):
    g = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([g.choice(N, size=min(n, N), replace=False),
                                     np.arange(max(0, N - 40), N)]))
    return rows


@pytest.fixture(scope="module")
def lm_head_weights():
    N, K = LM_HEAD_SHAPE
    W = torch_bf16_weights((N, K), 1300, "cuda:0")
    rows = sampled_rows(N, 3000, 1302)
    w_rows = host(W[torch.from_numpy(rows).to("cuda:0")].contiguous())
    return W, rows, w_rows


@pytest.mark.parametrize("R", [1, 4, 8, 12, 16, 17, 24])
def test_lm_head_sampled_rows(lm_head_weights, R):
    """The 151936 x 4096 LM head at every tile configuration it takes (32-row
    tiles up to 8 rows, 128-row tiles at 9-16, two column tiles above 16)."""
    W, rows, w_rows = lm_head_weights
    x = np.random.default_rng(1301 + R).standard_normal((R, W.shape[1])).astype(np.float32)
    X = dev(x)
    y = host(vs.verify_gemv_rows(W, X))
    ref, s = gemv_rows(w_rows, x)
    err = np.abs(y[:, rows].astype(np.float64) - ref)
    assert (err <= TOL * s).all()
    y1 = host(vs.verify_gemv_rows(W, X[R - 1:R]))
    assert np.array_equal(y1[0].view(np.uint32), y[R - 1].view(np.uint32))


@pytest.mark.parametrize("R", [1, 2, 4, 8, 16, 24])
def test_stack_layer_shapes_sampled_rows(R):
    """The fused shapes streamed in the 36-layer pass (qkv, o, gate|up, down)."""
    for i, (name, (N, K)) in enumerate(LAYER_SHAPES_FUSED.items()):
        W = torch_bf16_weights((N, K), 1400 + i, "cuda:0")
        x = np.random.default_rng(1410 + i).standard_normal((R, K)).astype(np.float32)
        X = dev(x)
        y = host(vs.verify_gemv_rows(W, X))
        rows = sampled_rows(N, 1500, 1420 + i)
        w_rows = host(W[torch.from_numpy(rows).to("cuda:0")].contiguous())
        ref, s = gemv_rows(w_rows, x)
        err = np.abs(y[:, rows].astype(np.float64) - ref)
        assert (err <= TOL * s).all(), name
        y1 = host(vs.verify_gemv_rows(W, X[R - 1:R]))
        assert np.array_equal(y1[0].view(np.uint32), y[R - 1].view(np.uint32)), name


def test_repeat_runs_are_bitwise_equal():
    w, x = gemv_case(1500, 4096, 4096, 8)
    W, X = dev(w), dev(x)
    a = host(vs.verify_gemv_rows(W, X))
    for _ in range(3):
        assert np.array_equal(host(vs.verify_gemv_rows(W, X)).view(np.uint32), a.view(np.uint32))


def test_strided_operands():
    """Leading dimensions larger than the row length (views into wider buffers)."""
    w, x = gemv_case(1600, 300, 264, 5)
    wide_w = np.zeros((300, 272), dtype=np.uint16)
    wide_w[:, :264] = w
    wide_x = np.zeros((5, 268), dtype=np.float32)
    wide_x[:, :264] = x
    W = dev(wide_w)[:, :264]
    X = dev(wide_x)[:, :264]
    Y = torch.full((5, 310), -7.0, device="cuda:0")
    vs.verify_gemv_rows(W, X, Y[:, :300])
    y = host(Y)
    check(y[:, :300], w, x)
    assert (y[:, 300:] == -7.0).all()


@pytest.mark.parametrize("N,K", [(65573, 1064), (6151, 4104), (24576, 4096), (24580, 4096),
                                 (4096, 12288), (4100, 12288), (4096, 12296), (6144, 4096),
                                 (6150, 4096)])
def test_shared_activation_paths_bit_identical(N, K):
    """Partitions across workgroups with a workspace of partial sums: long
    rows of >= 48 MB from 9 rows (the staged split-K kernel, 32-row tiles,
    for 4096 and 4100 x 12288; the older shared kernel for 4096 x 12296,
    whose k-blocks do not fit the staged kernels), other matrices of
    >= 48 MB below 65536 rows above 16 rows (staged split-K: 16-row tiles
    for 6144 and 6150 x 4096, 32-row tiles for 24576 and 24580 x 4096), and
    wider matrices of >= 48 MB whose k-blocks do not fit the staged kernels
    above 16 rows (all-K sharing); below those row counts the staged
    row-block kernel runs.  Their rows equal the 1-row call bit for bit,
    with the workspace and without it, and match the oracle.  Ragged N and a
    partial last k-block are included."""
    W = torch_bf16_weights((N, K), 3000 + N % 97 + K % 89, "cuda:0")
    x = np.random.default_rng(3100 + N % 97).standard_normal((24, K)).astype(np.float32)
    X = dev(x)
    single = np.stack([host(vs.verify_gemv_rows(W, X[r:r + 1]))[0] for r in range(24)])
    for R in (9, 12, 16, 17, 24):
        y = host(vs.verify_gemv_rows(W, X[:R].contiguous()))
        assert np.array_equal(y.view(np.uint32), single[:R].view(np.uint32)), f"R={R}"
        y0 = host(vs.verify_gemv_rows(W, X[:R].contiguous(), workspace=None))
        assert np.array_equal(y0.view(np.uint32), y.view(np.uint32)), f"R={R} without workspace"
    rows = sampled_rows(N, 800, 3200 + N % 97)
    w_rows = host(W[torch.from_numpy(rows).to("cuda:0")].contiguous())
    ref, s = gemv_rows(w_rows, x)
    err = np.abs(y[:, rows].astype(np.float64) - ref)
    assert (err <= TOL * s).all()


@pytest.mark.parametrize("N,K", [(4100, 4096), (6150, 4096), (70001, 2048), (1000, 12288),
                                 (17, 4096)])
def test_staged_row_block_ragged_rows(N, K):
    """Up to 16 rows (below 6144 matrix rows, and for wide matrices, at any
    R) the row-block kernel stages row runs through LDS; wide matrices take
    32-row tiles up to 8 rows, 128-row tiles up to 16 and 64-row tiles with
    two column tiles above.  Ragged N exercises the clamped rows.  Matches
    the oracle on sampled rows, and rows equal 1-row calls bit for bit up to
    24 rows."""
    W = torch_bf16_weights((N, K), 3300 + N % 101, "cuda:0")
    x = np.random.default_rng(3310 + N % 101).standard_normal((24, K)).astype(np.float32)
    X = dev(x)
    single = np.stack([host(vs.verify_gemv_rows(W, X[r:r + 1]))[0] for r in range(24)])
    for R in (2, 4, 8, 12, 24):
        y = host(vs.verify_gemv_rows(W, X[:R].contiguous()))
        assert np.array_equal(y.view(np.uint32), single[:R].view(np.uint32)), f"R={R}"
    rows = sampled_rows(N, 600, 3320 + N % 101)
    w_rows = host(W[torch.from_numpy(rows).to("cuda:0")].contiguous())
    ref, s = gemv_rows(w_rows, x[:8])
    y8 = host(vs.verify_gemv_rows(W, X[:8].contiguous()))
    err = np.abs(y8[:, rows].astype(np.float64) - ref)
    assert (err <= TOL * s).all()


def test_workspace_fallbacks_and_stale_contents():
    """The split-K path's workspace: a buffer one byte too small or
    misaligned selects the single-launch path, and a workspace holding stale
    bytes (all 0xFF, NaN as fp32) is simply overwritten; every variant gives
    the same bits as the call with a fresh workspace."""
    N, K, R = 4096, 12288, 12  # long rows: split-K from 9 rows
    W = torch_bf16_weights((N, K), 3400, "cuda:0")
    X = dev(np.random.default_rng(3401).standard_normal((R, K)).astype(np.float32))
    need = vs.verify_gemv_rows_workspace_bytes(N, K, R)
    assert need > 0
    ref = host(vs.verify_gemv_rows(W, X))
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda:0")
    big = torch.empty(need + 64, dtype=torch.uint8, device="cuda:0")
    stale = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda:0")
    for ws in (small, big[4:4 + need], stale, None):
        y = host(vs.verify_gemv_rows(W, X, workspace=ws))
        assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


FAMILY_CASES = [(fam, name) for fam, shapes in FAMILY_SHAPES.items() if fam != "hidden4096"
                for name in shapes]


@pytest.mark.parametrize("fam,name", FAMILY_CASES)
def test_other_model_sizes_sampled_rows(fam, name):
    """The fused projections and LM heads of the hidden-2560 and hidden-5120
    models at every kernel and tile configuration the dispatch picks for
    them (row-block and split-K, one and two column tiles), on sampled
    output rows against the oracle, with the last row equal to its 1-row call."""
    N, K = FAMILY_SHAPES[fam][name]
    W = torch_bf16_weights((N, K), 1600 + N % 997 + K % 89, "cuda:0")
    rows = sampled_rows(N, 1200, 1601 + N % 991)
    w_rows = host(W[torch.from_numpy(rows).to("cuda:0")].contiguous())
    for R in (1, 4, 8, 9, 16, 17, 24):
        x = np.random.default_rng(1602 + R + K).standard_normal((R, K)).astype(np.float32)
        X = dev(x)
        y = host(vs.verify_gemv_rows(W, X))
        ref, s = gemv_rows(w_rows, x)
        err = np.abs(y[:, rows].astype(np.float64) - ref)
        assert (err <= TOL * s).all(), (fam, name, R)
        y1 = host(vs.verify_gemv_rows(W, X[R - 1:R]))
        assert np.array_equal(y1[0].view(np.uint32), y[R - 1].view(np.uint32)), (fam, name, R)


@pytest.mark.parametrize("N,K,R", [(64, 256, 4), (1000, 1000, 5), (4096, 4096, 9), (6144, 4096, 17)])
def test_non_finite_and_subnormal_activations(N, K, R):
    """Activations with +-inf, opposite infinities, NaN, and rows scaled into
    the subnormal range, against the oracle's term-by-term IEEE reading:
    NaN exactly where it is NaN, the same infinities, and finite outputs
    within the tolerance plus the library's absolute term 2^-133 * sum|w|
    (a subnormal activation keeps its bits down to 2^-133, the smallest bf16
    subnormal; its three-plane split cannot hold the rest) and K * 2^-149
    (the resolution of fp32 sums in that range).  Row identity holds for
    every row."""
    w, x = gemv_case(1700 + N + R, N, K, R)
    x[0, 3] = np.inf                     # +inf: +-inf outputs, NaN where w = 0
    x[1, 5], x[1, 9] = -np.inf, np.inf   # opposite infinities: NaN or +-inf by the weights' signs
    x[2, 7] = np.nan
    x[3] *= np.float32(2.0 ** -130)      # subnormal activations
    if R > 4:
        x[4] *= np.float32(2.0 ** -120)  # small normal activations, subnormal products
    W, X = dev(w), dev(x)
    y = host(vs.verify_gemv_rows(W, X))
    ref, s = gemv_rows(w, x)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(y), nan)
    inf = np.isinf(ref)
    assert np.array_equal(y[inf], ref[inf])
    fin = ~(nan | inf)
    _, sw = gemv_rows(w, np.ones((1, K), dtype=np.float32))   # sum_k |w[n][k]|
    bound = TOL * s + np.broadcast_to(sw, s.shape) * 2.0 ** -133 + K * 2.0 ** -149
    err = np.abs(y[fin].astype(np.float64) - ref[fin])
    assert (err <= bound[fin]).all(), float((err / bound[fin]).max())
    assert np.abs(ref[3]).max() > 0 and np.abs(y[3]).max() > 0   # not flushed to zero
    for r in range(R):
        y1 = host(vs.verify_gemv_rows(W, X[r:r + 1]))
        assert np.array_equal(y1[0].view(np.uint32), y[r].view(np.uint32)), r
