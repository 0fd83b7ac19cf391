"""topk_rows_noalloc (the allocation-free top-K for callers that cannot
allocate) against topk_rows with a caller workspace, through the C ABI.

Outputs must be byte-identical (values and indices), on consecutive calls
that reuse the library's fixed per-GPU scratch area: first a larger input,
then a smaller one, so that the second call runs over stale scratch
contents left by the first.  Inputs carry planted ties, 1-ulp neighbours,
NaN, -inf and +-0 (the draft-row construction).
"""

from __future__ import annotations

import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def run_pair(lib, torch, x, K):
    """(noalloc vals, idx), (topk_rows vals, idx) for x [rows][V] on the GPU."""
    dev = x.device
    rows, V = x.shape
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for mode in ("noalloc", "workspace"):
        vals = torch.full((rows, K), 7.0, dtype=torch.float32, device=dev)
        idx = torch.full((rows, K), -7, dtype=torch.int32, device=dev)
        if mode == "noalloc":
            st = lib.topk_rows_noalloc(x.data_ptr(), x.stride(0), rows, V, K, vals.data_ptr(),
                                       idx.data_ptr(), K, stream)
        else:
            nws = lib.topk_rows_workspace_bytes(rows, V, K)
            ws = torch.empty(max(16, nws), dtype=torch.uint8, device=dev)
            st = lib.topk_rows(x.data_ptr(), x.stride(0), rows, V, K, vals.data_ptr(), idx.data_ptr(),
                               K, ws.data_ptr(), nws, stream)
        assert st == 0, (mode, st)
        torch.cuda.synchronize()
        outs.append((vals.cpu().numpy(), idx.cpu().numpy()))
    return outs


def same(a, b):
    (va, ia), (vb, ib) = a, b
    return np.array_equal(va.view(np.uint32), vb.view(np.uint32)) and np.array_equal(ia, ib)


def test_noalloc_matches_topk_rows_on_consecutive_calls():
    import torch

    import synth
    import verify_sampling_amd as vs

    lib = vs.library()
    dev = "cuda:0"
    V = synth.VOCAB
    big = torch.from_numpy(synth.topk_planted_rows(8400, rows=24, vocab=V, K=64)).to(dev)
    small = torch.from_numpy(synth.topk_planted_rows(8401, rows=5, vocab=V, K=16)).to(dev)
    print("scratch bytes used: big", lib.topk_rows_workspace_bytes(24, V, 64),
          "small", lib.topk_rows_workspace_bytes(5, V, 16), flush=True)
    a, b = run_pair(lib, torch, big, 64)
    assert same(a, b)
    a, b = run_pair(lib, torch, small, 16)   # second call, smaller input, stale scratch
    assert same(a, b)
    # a third call with a different chunking (4096-element chunks: a batch of rows)
    batch = torch.from_numpy(synth.logits(8402, (600, 9000))).to(dev)
    a, b = run_pair(lib, torch, batch, 64)
    assert same(a, b)
    # rows of one chunk (no scratch used) and K = 1
    one = torch.from_numpy(synth.logits(8403, (7, 1000))).to(dev)
    a, b = run_pair(lib, torch, one, 1)
    assert same(a, b)


def test_noalloc_refuses_inputs_beyond_its_scratch():
    import torch

    import verify_sampling_amd as vs

    lib = vs.library()
    V, rows, K = 151936, 256, 64
    assert lib.topk_rows_workspace_bytes(rows, V, K) > lib.topk_rows_noalloc_max_scratch_bytes()
    x = torch.zeros((rows, V), dtype=torch.float32, device="cuda:0")
    out = torch.zeros((rows, K), dtype=torch.float32, device="cuda:0")
    idx = torch.zeros((rows, K), dtype=torch.int32, device="cuda:0")
    st = lib.topk_rows_noalloc(x.data_ptr(), V, rows, V, K, out.data_ptr(), idx.data_ptr(), K,
                               torch.cuda.current_stream().cuda_stream)
    assert st == -8
    torch.cuda.synchronize()
    assert int(idx.abs().sum()) == 0  # nothing was launched
    with pytest.raises(vs.VerifySamplingError):
        vs.topk_rows_noalloc(x, K)


def test_noalloc_binding_matches_the_oracle_on_sampled_rows():
    import torch

    import synth
    import verify_sampling_amd as vs
    from oracle.topk import topk_rows

    x = synth.topk_planted_rows(8404, rows=6, vocab=synth.VOCAB, K=16)
    v, i = vs.topk_rows_noalloc(torch.from_numpy(x).to("cuda:0"), 16)
    torch.cuda.synchronize()
    for r in (0, 3, 5):
        ov, oi = topk_rows(x[r:r + 1], 16)
        assert np.array_equal(i.cpu().numpy()[r], oi[0])
        assert np.array_equal(v.cpu().numpy()[r].view(np.uint32), ov[0].view(np.uint32))
