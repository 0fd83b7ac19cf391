"""GPU parity of topk_rows: byte identity with the oracle's pool order.

Planted ties straddling rank K, 1-ulp neighbours, duplicated maxima, NaN,
-inf and +-0 follow the byte-identity gate described under "Code map" of
"feat(dflash): developer-only online draft tuning".
"""

import numpy as np
import pytest

import verify_sampling_amd as vs
from gpu_common import dev, host
from oracle.topk import topk_rows
from synth import VOCAB, logits, topk_planted_rows

pytestmark = pytest.mark.gpu


def compare(x, K):
    vals, idx = vs.topk_rows(dev(x), K)
    gv, gi = host(vals), host(idx)
    ov, oi = topk_rows(x, K)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv.view(np.uint32), ov.view(np.uint32))


def test_draft_rows_top16_planted():
    compare(topk_planted_rows(1500, rows=15, vocab=VOCAB, K=16), 16)


def test_pool_top64_target_rows():
    compare(logits(1501, (4, VOCAB)), 64)


def test_argmax_k1():
    compare(topk_planted_rows(1502, rows=6, vocab=VOCAB, K=1), 1)


@pytest.mark.parametrize("V,K", [(64, 64), (100, 1), (100, 16), (4096, 64), (4097, 64),
                                 (8191, 7), (12289, 64), (262144, 64)])
def test_sizes_and_ragged_chunks(V, K):
    x = logits(1503 + V + K, (3, V))
    x[1, :] = np.float32(0.5)           # all equal: lowest indices
    x[2, : V // 2] = np.nan             # half NaN, the rest ordinary
    compare(x, K)


@pytest.mark.parametrize("K", [64, 16, 1])
def test_narrow_bands_and_minus_inf_thresholds(K):
    """Rows whose thresholds take the search's corner cases: distinct values
    packed within 2^-6 of each other (the first threshold's coarse bits
    leave most of a chunk above it, so its search goes on to the low bits),
    and chunks whose K-th largest group maximum is -inf (a threshold with
    cleared low bits would fall among NaN patterns below -inf's key)."""
    V = VOCAB
    rng = np.random.default_rng(1510 + K)
    x = np.empty((5, V), dtype=np.float32)
    band = (np.float32(1.0) + rng.permutation(V).astype(np.float32) * np.float32(2.0 ** -23))
    x[0] = band                                   # 1 + i * 2^-23, distinct, in [1, 1.02)
    x[1] = -band                                  # the same band, negative
    x[2] = -np.inf                                # a few finite values per 1024, the rest -inf
    x[2, rng.choice(V, V // 200, replace=False)] = rng.standard_normal(V // 200).astype(np.float32)
    x[3] = np.where(rng.random(V) < 0.5, np.float32(np.nan), np.float32(-np.inf))
    x[3, rng.choice(V, 40, replace=False)] = np.float32(2.0)
    x[4] = np.where(rng.random(V) < 0.5, band, np.float32(-np.inf))
    compare(x, K)


def random_rows(rng, rows, V):
    """Rows of mixed kinds for the randomized parity test: ordinary logits,
    narrow bands of distinct values, integers (many exact ties),
    bf16-rounded values, mostly -inf, NaN mixes, plateaus with a few values
    above them, and all-equal rows."""
    x = np.empty((rows, V), dtype=np.float32)
    for r in range(rows):
        kind = int(rng.integers(0, 8))
        if kind == 0:
            row = rng.standard_normal(V).astype(np.float32) * np.float32(rng.uniform(0.5, 8.0))
        elif kind == 1:
            row = (np.float32(rng.uniform(-4, 4)) + rng.permutation(V).astype(np.float32)
                   * np.float32(2.0 ** -int(rng.integers(16, 24))))
        elif kind == 2:
            row = rng.integers(-20, 20, size=V).astype(np.float32)
        elif kind == 3:
            b = rng.standard_normal(V).astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
            row = b.view(np.float32)
        elif kind == 4:
            row = np.full(V, -np.inf, dtype=np.float32)
            n = int(rng.integers(0, min(V, 200) + 1))
            row[rng.choice(V, n, replace=False)] = rng.standard_normal(n).astype(np.float32)
        elif kind == 5:
            row = rng.standard_normal(V).astype(np.float32)
            row[rng.random(V) < rng.uniform(0.1, 0.9)] = np.nan
            row[rng.random(V) < 0.05] = -np.inf
        elif kind == 6:
            row = np.full(V, np.float32(rng.uniform(-2, 2)), dtype=np.float32)
            n = int(rng.integers(0, min(V, 100)))
            row[rng.choice(V, n, replace=False)] += np.abs(rng.standard_normal(n)).astype(np.float32) + 1
        else:
            row = np.full(V, np.float32(rng.choice([0.0, -0.0, 1.5, -3.25])), dtype=np.float32)
        x[r] = row
    return x


@pytest.mark.parametrize("seed", range(1520, 1544))
def test_random_rows_against_oracle(seed):
    """Seeded random sizes, K and row kinds; exact ids and value bits."""
    rng = np.random.default_rng(seed)
    V = int(rng.choice([64, 1000, 4096, 5000, 50257, 151936, 151936, 262144]))
    K = int(rng.integers(1, min(V, 64) + 1))
    rows = int(rng.integers(1, 16))
    x = random_rows(rng, rows, V)
    print(f"seed {seed}: rows={rows} V={V} K={K}", flush=True)
    compare(x, K)


@pytest.mark.parametrize("K", [64, 23])
def test_random_rows_batched_against_oracle(K):
    """64 rows of 151936 in mixed kinds: enough chunks for the 4096-element
    chunk stage."""
    rng = np.random.default_rng(1550 + K)
    x = random_rows(rng, 64, VOCAB)
    compare(x, K)


def test_special_rows():
    V = 5000
    x = logits(1504, (5, V))
    x[0, :] = -np.inf
    x[1, :] = np.nan
    x[2, :] = -0.0
    x[2, ::7] = 0.0
    x[3, :] = np.inf
    x[3, 10] = np.nan
    x[4, ::3] = -np.inf
    compare(x, 64)


def test_strided_input_and_output():
    x = logits(1505, (3, 9000))
    wide = np.full((3, 9100), 99.0, dtype=np.float32)
    wide[:, :9000] = x
    X = dev(wide)[:, :9000]
    import torch
    ov = torch.zeros((3, 80), dtype=torch.float32, device="cuda:0")
    oi = torch.zeros((3, 80), dtype=torch.int32, device="cuda:0")
    vs.topk_rows(X, 64, ov[:, :64], oi[:, :64])
    rv, ri = topk_rows(x, 64)
    assert np.array_equal(host(oi)[:, :64], ri)
    assert (host(oi)[:, 64:] == 0).all()


def test_repeat_runs_are_identical():
    x = topk_planted_rows(1506, rows=15, vocab=VOCAB, K=16)
    X = dev(x)
    a = host(vs.topk_rows(X, 16)[1])
    for _ in range(3):
        assert np.array_equal(host(vs.topk_rows(X, 16)[1]), a)


def crafted_dense_lanes(V=4096):
    """A row whose top values sit in 16 of the 64 lanes of the wavefront layout,
    so the group-maxima threshold passes 784 keys and the exact radix select
    of the batched kernel runs."""
    x = np.full(V, -5.0, dtype=np.float32)
    i = np.arange(V)
    lane = (i % 256) // 4
    j = 4 * (i // 256) + i % 4
    x[lane < 16] = 1000.0 + j[lane < 16]
    return x


def test_batched_rows_wave_kernel():
    """2048 rows x 4096: the throughput kernel (one wavefront per row)."""
    rows = 2048
    x = logits(1510, (rows, 4096))
    x[1] = crafted_dense_lanes()
    x[2] = 0.75                       # all equal
    x[3] = np.arange(4096, dtype=np.float32)
    x[4, ::5] = np.nan
    x[5, :4000] = -np.inf
    x[6, ::3] = x[6, 0]               # ties
    x[7] = crafted_dense_lanes()[::-1].copy()
    compare(x, 64)


def test_batched_multi_chunk_rows_wave_kernel():
    """1024 rows x 8292 (three chunks, the last ragged): stage 1 by wavefront, then stage 2."""
    rows = 1024
    x = logits(1511, (rows, 8292))
    x[0, :4096] = crafted_dense_lanes()
    x[1, :] = 3.0
    x[2, 8190:] = 1e30                # maxima in the ragged chunk
    compare(x, 16)


def compare_rows(x, K, check):
    """Runs the whole batch on the GPU; the oracle checks the listed rows."""
    vals, idx = vs.topk_rows(dev(x), K)
    gv, gi = host(vals), host(idx)
    ov, oi = topk_rows(x[check], K)
    assert np.array_equal(gi[check], oi)
    assert np.array_equal(gv[check].view(np.uint32), ov.view(np.uint32))


def from_bits(b):
    return np.asarray(b, dtype=np.uint32).view(np.float32)


def special_batch(seed, rows=2048, V=4096):
    g = np.random.default_rng(seed)
    x = logits(seed, (rows, V))
    # distinct denormals of both signs: the threshold comparison runs on them
    mag = g.choice(np.arange(1, 1 << 23, dtype=np.uint32), size=V, replace=False)
    sign = (g.random(V) < 0.5).astype(np.uint32) << np.uint32(31)
    x[0] = from_bits(mag | sign)
    x[1] = x[0]
    x[1, ::2] = 0.0
    x[1, 1::4] = -0.0
    # signalling and negative NaN bit patterns among ordinary values
    x[2, ::7] = from_bits(0x7F800001)
    x[3, ::5] = from_bits(0xFFC00000)
    x[4, 3::11] = from_bits(0x7FBFFFFF)
    x[4, 5::13] = from_bits(0xFF800001)
    # NaN apart from a few numbers: fewer than K group maxima are numbers
    x[5] = np.nan
    x[5, [5, 900, V - 1]] = [1.0, -2.0, 3.0]
    x[6] = np.nan
    x[6, g.choice(V, 100, replace=False)] = g.standard_normal(100).astype(np.float32)
    x[7] = np.nan
    x[8] = -np.inf
    x[8, 17] = np.nan
    # 70 copies of +inf: ties at the top, ordered by index
    x[9, g.choice(V, 70, replace=False)] = np.inf
    # values spread over one lane's groups only
    x[10] = -1.0
    x[10, 4 * 9 + 256 * np.arange(16)[:, None] + np.arange(4)[None, :]] = np.arange(64).reshape(16, 4)
    return x


@pytest.mark.parametrize("K", [64, 16, 7, 1])
def test_batched_wave_kernel_special_values(K):
    """Denormals, NaN bit patterns, NaN-dominated rows and ties through the
    wavefront kernel (2048 rows x 4096); the oracle checks the crafted rows
    and a sample of the ordinary ones."""
    x = special_batch(1512)
    check = np.r_[0:16, 16:2048:97]
    compare_rows(x, K, check)


@pytest.mark.parametrize("V,K", [(4106, 64), (4196, 64), (4196, 16), (8192, 64)])
def test_batched_wave_kernel_ragged_last_chunk(V, K):
    """1024 rows of two chunks; the last one holds 10 or 100 elements (fewer
    group maxima than K, or fewer elements than K) or is full."""
    x = logits(1513 + V + K, (1024, V))
    x[0, :4096] = np.nan
    x[1, 4096:] = 1e30
    x[2, :] = 2.0
    check = np.r_[0:8, 8:1024:61]
    compare_rows(x, K, check)


def crafted_lane_block(n):
    """Values for a 1024-element chunk (its first n valid) whose largest values
    sit in lanes 0-31 of the 16-values-per-lane layout, with distinct group
    maxima: for K = 64 about 160 elements pass the group-maxima threshold
    (the widest ranking)."""
    i = np.arange(n)
    lane = (i % 256) // 4
    j = 4 * (i // 256) + i % 4
    out = np.full(n, np.nan, dtype=np.float32)
    sel = lane < 32
    out[sel] = (1000.0 + j[sel] + 0.001 * lane[sel]).astype(np.float32)
    return out, sel


@pytest.mark.parametrize("K", [64, 16, 5])
def test_few_rows_fallbacks_and_ties(K):
    """A handful of long rows (1024-element chunks, then the merge): crowded
    lanes in a full and in the ragged last chunk, exact ties over every chunk
    (the merge's continuation for K = 16 and its second round for K = 64),
    and NaN chunks with a few numbers (every element survives the group
    maxima, so the chunk stage's exact threshold runs)."""
    V = VOCAB
    x = logits(1520 + K, (5, V))
    x[3, :3072] = np.nan
    x[3, [7, 1500, 2049, 3000]] = [1.0, -np.inf, 0.0, 2.5]
    blk, sel = crafted_lane_block(1024)
    x[0, :1024][sel] = blk[sel]
    last = (V // 1024) * 1024
    blk, sel = crafted_lane_block(V - last)
    x[1, last:][sel] = blk[sel]
    x[2] = np.random.default_rng(1525).integers(0, 10, V).astype(np.float32)
    compare(x, K)


@pytest.mark.parametrize("rows", [53, 54])
def test_chunking_boundary(rows):
    """53 rows of 151936 take 1024-element chunks, 54 rows take 4096-element
    chunks; both give the oracle's result."""
    x = logits(1530 + rows, (rows, VOCAB))
    x[0] = 1.5
    x[1] = np.random.default_rng(1531).integers(0, 4, VOCAB).astype(np.float32)
    x[2, ::2] = np.nan
    compare_rows(x, 64, np.r_[0:4, rows - 2:rows])


@pytest.mark.parametrize("K", [10, 12, 14, 16])
def test_crowded_rows_read_full_chunks_to_the_end(K):
    """Rows whose top K crowds into the first 1024-element chunks (equal
    values, mostly -inf with a few numbers, a few distinct values over the
    whole row): the merge reads those chunks past their first 8 entries in
    one more round; the pool must still be the oracle's, byte for byte."""
    V = VOCAB
    g = np.random.default_rng(1540 + K)
    x = logits(1541 + K, (4, V))
    x[0, :] = np.float32(-3.5)
    x[1, :] = -np.inf
    x[1, g.choice(V, size=K // 2, replace=False)] = g.standard_normal(K // 2).astype(np.float32)
    x[2] = g.integers(0, 3, V).astype(np.float32)
    x[3, : 5 * 1024] = np.float32(1e4)   # five whole chunks of the row maximum
    compare(x, K)
