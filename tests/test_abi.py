"""The C-ABI library loads, exports every symbol the header declares, and
rejects invalid arguments on the host before anything is launched.

No call here launches a kernel, so this runs without a GPU.
"""

import ctypes
import os
import re

import pytest

import verify_sampling_amd as vs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "verify_sampling.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = vs.library()
    names = declared_functions()
    assert set(names) == set(vs.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    lib = vs.library()
    assert lib.vs_abi_version() == 6
    assert lib.vs_status_string(0) == b"ok"
    for code in range(-8, 0):
        assert lib.vs_status_string(code) != b"unknown status"
    assert lib.vs_last_error_detail() == b""


FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first


def test_gemv_rejects_before_launch():
    lib = vs.library()
    assert lib.verify_gemv_rows(None, 8, 4, 8, FAKE, 8, 1, FAKE, 4, None, 0, None) == -1
    assert lib.verify_gemv_rows(FAKE, 8, 4, 8, FAKE, 8, 0, FAKE, 4, None, 0, None) == -2      # R = 0
    assert lib.verify_gemv_rows(FAKE, 8, 4, 8, FAKE, 8, 25, FAKE, 4, None, 0, None) == -2     # R > 24
    assert lib.verify_gemv_rows(FAKE, 12, 4, 12, FAKE, 12, 1, FAKE, 4, None, 0, None) == -2   # K % 8
    assert lib.verify_gemv_rows(FAKE, 8, 4, 8, FAKE, 8, 1, FAKE, 3, None, 0, None) == -2      # ldy < N
    assert lib.verify_gemv_rows(FAKE, 1 << 24, 4, 8, FAKE, 8, 1, FAKE, 4, None, 0, None) == -2  # ldw >= 2^24
    assert lib.verify_gemv_rows(FAKE, 8, 4, 8, FAKE, 1 << 24, 1, FAKE, 4, None, 0, None) == -2  # ldx >= 2^24
    assert lib.verify_gemv_rows(ctypes.c_void_p(0x100008), 8, 4, 8, FAKE, 8, 1, FAKE, 4, None, 0, None) == -6
    # the workspace is optional; its size is zero where no path uses one
    assert lib.verify_gemv_rows_workspace_bytes(4096, 4096, 4) == 0
    assert lib.verify_gemv_rows_workspace_bytes(151936, 4096, 24) == 0
    assert lib.verify_gemv_rows_workspace_bytes(4096, 12288, 4) == 0
    # partitions across workgroups: long rows of >= 48 MB from 9 rows, other
    # matrices of >= 48 MB below 65536 rows above 16 rows, and wider ones of
    # >= 48 MB above 16 rows only where the staged kernels cannot run
    # (K % 32 != 0)
    assert lib.verify_gemv_rows_workspace_bytes(4096, 12288, 8) == 0
    assert lib.verify_gemv_rows_workspace_bytes(4096, 12288, 9) == 16 * 9 * 4096 * 4
    assert lib.verify_gemv_rows_workspace_bytes(4096, 12288, 16) == 16 * 16 * 4096 * 4
    assert lib.verify_gemv_rows_workspace_bytes(4096, 12296, 8) == 0
    assert lib.verify_gemv_rows_workspace_bytes(4096, 12296, 9) == 16 * 9 * 4096 * 4
    assert lib.verify_gemv_rows_workspace_bytes(6144, 4096, 16) == 0
    assert lib.verify_gemv_rows_workspace_bytes(6144, 4096, 17) == 8 * 17 * 6144 * 4
    assert lib.verify_gemv_rows_workspace_bytes(6144, 4096, 24) == 8 * 24 * 6144 * 4
    assert lib.verify_gemv_rows_workspace_bytes(24576, 4096, 16) == 0
    assert lib.verify_gemv_rows_workspace_bytes(24576, 4096, 24) == 4 * 24 * 24576 * 4
    assert lib.verify_gemv_rows_workspace_bytes(151936, 4096, 24) == 0
    assert lib.verify_gemv_rows_workspace_bytes(4096, 4096, 24) == 0
    assert lib.verify_gemv_rows_workspace_bytes(6152, 4104, 16) == 0
    assert lib.verify_gemv_rows_workspace_bytes(6152, 4104, 17) == 8 * 17 * 6152 * 4
    # 4096 x 12288 at 24 rows: 16 K partitions of 24 x 4096 fp32 partial sums
    assert lib.verify_gemv_rows_workspace_bytes(4096, 12288, 24) == 16 * 24 * 4096 * 4
    assert lib.verify_gemv_rows_workspace_bytes(4096, 12288, 25) == 0


def test_topk_rejects_before_launch():
    lib = vs.library()
    assert lib.topk_rows(FAKE, 100, 1, 100, 65, FAKE, FAKE, 65, None, 0, None) == -2   # K > 64
    assert lib.topk_rows(FAKE, 10, 1, 10, 11, FAKE, FAKE, 11, None, 0, None) == -2     # K > V
    # a few long rows take 1024-element chunks, batches 4096-element ones
    assert lib.topk_rows_workspace_bytes(4, 151936, 64) == 4 * 149 * 64 * 8
    assert lib.topk_rows_workspace_bytes(53, 151936, 16) == 53 * 149 * 16 * 8
    assert lib.topk_rows_workspace_bytes(54, 151936, 64) == 54 * 38 * 64 * 8
    assert lib.topk_rows_workspace_bytes(4, 1024, 64) == 0
    assert lib.topk_rows_workspace_bytes(4, 4096, 64) == 0
    assert lib.topk_rows(FAKE, 8192, 1, 8192, 8, FAKE, FAKE, 8, None, 0, None) == -5   # workspace


def test_topk_noalloc_rejects_before_launch():
    """The allocation-free top-K checks its arguments like topk_rows and
    refuses inputs whose per-chunk lists exceed its fixed 4 MiB scratch
    area, before touching the GPU."""
    lib = vs.library()
    assert lib.topk_rows_noalloc_max_scratch_bytes() == 4 << 20
    assert lib.topk_rows_noalloc(None, 100, 1, 100, 8, FAKE, FAKE, 8, None) == -1
    assert lib.topk_rows_noalloc(FAKE, 100, 1, 100, 65, FAKE, FAKE, 65, None) == -2   # K > 64
    assert lib.topk_rows_noalloc(FAKE, 100, 1, 100, 8, FAKE, FAKE, 7, None) == -2     # ld_out < K
    # 54 rows of 151936 at K = 64 need 54 * 38 chunks * 64 * 8 bytes = 1.0 MiB: fits;
    # 256 rows need 4.75 MiB: refused
    assert lib.topk_rows_workspace_bytes(54, 151936, 64) < 4 << 20
    assert lib.topk_rows_workspace_bytes(256, 151936, 64) > 4 << 20
    assert lib.topk_rows_noalloc(FAKE, 151936, 256, 151936, 64, FAKE, FAKE, 64, None) == -8


def test_policy_and_penalty_and_accept_reject_before_launch():
    lib = vs.library()
    assert lib.sample_policy_rows(FAKE, FAKE, 65, 1, 65, 0.7, 20, 0.9, 0.1, FAKE, FAKE, FAKE, 65,
                                  None, None, None) == -2
    assert lib.sample_policy_rows(FAKE, FAKE, 8, 1, 8, float("nan"), 20, 0.9, 0.1, FAKE, FAKE, FAKE,
                                  8, None, None, None) == -3
    assert lib.sample_policy_rows(FAKE, FAKE, 8, 1, 8, 0.7, 20, 0.9, 0.1, FAKE, FAKE, FAKE, 8,
                                  FAKE, None, None) == -1
    assert lib.penalize_rows(FAKE, None, 100, 1, 100, 100, FAKE, 4, None, 0, 5000, 1.1, 0, 0,
                             None) == -3   # window
    assert lib.penalize_rows(FAKE, None, 100, 1, 100, 100, FAKE, 4, None, 0, 64, 0.0, 0, 0,
                             None) == -3   # repeat <= 0
    assert lib.penalize_rows(FAKE, None, 100, 1, 99, 100, FAKE, 4, None, 0, 64, 1.1, 0, 0,
                             None) == -2   # dense width != vocab
    # tree rows: node count bounded, tokens and parent required when there are nodes
    assert lib.penalize_tree_rows(FAKE, None, 100, 100, 100, FAKE, 4, FAKE, FAKE, 64, 64, 1.1,
                                  0, 0, None) == -2
    assert lib.penalize_tree_rows(FAKE, None, 100, 100, 100, FAKE, 4, FAKE, None, 3, 64, 1.1,
                                  0, 0, None) == -1
    assert lib.penalize_tree_rows(FAKE, None, 100, 100, 100, None, 0, None, None, 0, 64, 1.1,
                                  0, 0, None) == 0
    # nothing to penalise: returns OK without launching
    assert lib.penalize_rows(FAKE, None, 100, 1, 100, 100, None, 0, None, 0, 64, 1.1, 0, 0,
                             None) == 0
    assert lib.spec_accept_rows(6, 1, 1, FAKE, None, None, 4, 2, None, None, None, 1, 1, FAKE,
                                None, None, FAKE, FAKE, None) == -3   # unknown mode
    # the naive tree walk needs parent[] when there are nodes
    assert lib.spec_accept_rows(5, 1, 1, FAKE, FAKE, FAKE, 4, 2, None, None, None, 1, 1, FAKE,
                                None, FAKE, FAKE, FAKE, None) == -1
    for mode in (3, 4, 5):   # point-mass and naive modes need p's probabilities and the uniforms
        assert lib.spec_accept_rows(mode, 1, 1, FAKE, None, FAKE, 4, 2, None, None, None, 1, 1,
                                    FAKE, None, FAKE, FAKE, FAKE, None) == -1
        assert lib.spec_accept_rows(mode, 1, 1, FAKE, FAKE, FAKE, 4, 2, None, None, None, 1, 1,
                                    FAKE, None, None, FAKE, FAKE, None) == -1
    assert lib.spec_accept_rows(0, 1, 64, FAKE, FAKE, FAKE, 4, 65, FAKE, FAKE, FAKE, 4, 64, FAKE,
                                None, FAKE, FAKE, FAKE, None) == -2   # k > 63
    assert lib.spec_accept_rows(0, 1, 2, FAKE, FAKE, FAKE, 4, 3, FAKE, FAKE, FAKE, 4, 2, FAKE,
                                None, None, FAKE, FAKE, None) == -1   # sampled needs u
    assert lib.spec_accept_rows(2, 1, 2, FAKE, None, None, 4, 3, None, None, None, 1, 0, FAKE,
                                None, None, FAKE, FAKE, None) == -1   # tree needs parent


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(vs, "_lib", None)
    with pytest.raises(vs.VerifySamplingError):
        vs.library(str(tmp_path / "missing.so"))


def test_tree_attention_rejects_before_launch():
    lib = vs.library()
    ws = lib.tree_attention_rows_workspace_bytes(25, 32, 8, 2080)
    assert ws > 0
    args = lambda **k: dict(dict(q=FAKE, R=25, Hq=32, D=128, kc=FAKE, vc=FAKE, L=4096, ctx=2080, ks=FAKE,
                                 vs=FAKE, S=25, par=FAKE, Hkv=8, scale=0.088, out=FAKE, ws=FAKE, nws=ws), **k)
    call = lambda a: lib.tree_attention_rows(a["q"], a["R"], a["Hq"], a["D"], a["kc"], a["vc"], a["L"], a["ctx"],
                                            a["ks"], a["vs"], a["S"], a["par"], a["Hkv"], a["scale"], a["out"],
                                            a["ws"], a["nws"], None)
    assert call(args(q=None)) == -1
    assert call(args(D=64)) == -4                       # head dimension 128 only
    assert call(args(R=65, S=65)) == -2                 # at most 64 tree rows
    assert call(args(Hq=30)) == -2                      # Hq % Hkv
    assert call(args(ctx=4097)) == -2                   # ctx_len > cache_len
    assert call(args(S=24)) == -2                       # scr_len < R
    assert call(args(scale=float("inf"))) == -3
    assert call(args(nws=ws - 1)) == -5
    assert call(args(R=64, S=64, Hq=16, Hkv=2)) == -2   # 8 heads x 64 rows > 256 queries per KV head
    assert lib.tree_commit_kv(FAKE, FAKE, 100, 90, FAKE, FAKE, 25, FAKE, 11, 8, 128, None) == -2  # past the cache
    assert lib.tree_commit_kv(FAKE, FAKE, 100, 90, FAKE, FAKE, 25, FAKE, 3, 8, 12, None) == -2    # D % 8
    assert lib.tree_commit_kv(FAKE, FAKE, 100, 90, FAKE, FAKE, 25, None, 0, 8, 128, None) == 0    # nothing to copy


def test_verify_tree_window_rejects_before_launch():
    lib = vs.library()
    V = 151936
    ws = lib.verify_window_workspace_bytes(25, V)
    base = dict(logits=FAKE, ld=V, R=25, V=V, ctx=FAKE, n_ctx=100, tokens=FAKE, parent=FAKE, window=64,
                rep=1.1, pres=1.5, freq=0.2, T=0.7, top_k=20, top_p=0.95, min_p=0.05, u=FAKE, pv=FAKE, pi=FAKE,
                di=FAKE, dp=FAKE, dl=FAKE, tok=FAKE, n=FAKE, ws=FAKE, nws=ws)

    def call(**kw):
        a = dict(base, **kw)
        return lib.verify_tree_window(*a.values(), None)

    assert call(logits=None) == -1
    assert call(R=0) == -2
    assert call(R=65) == -2                    # at most 64 rows (63 nodes)
    assert call(V=63) == -2
    assert call(ld=V - 1) == -2
    assert call(parent=None) == -1             # nodes need their parents
    assert call(tokens=None) == -1
    assert call(u=None) == -1                  # sampled walk draws
    assert call(window=5000) == -3
    assert call(rep=0.0) == -3
    assert call(T=float("nan")) == -3
    assert call(nws=ws - 1) == -5
    assert call(ctx=None) == -1


def test_verify_windows_rejects_before_launch():
    lib = vs.library()
    base = dict(p=FAKE, ldp=4096, q=FAKE, ldq=4096, B=16, k=3, V=4096, T=0.7, top_k=20, top_p=0.95,
                min_p=0.05, ud=FAKE, u=FAKE, drafts=FAKE, pi=FAKE, pp=FAKE, pl=FAKE, qi=FAKE, qp=FAKE,
                ql=FAKE, tok=FAKE, n=FAKE)

    def call(**kw):
        a = dict(base, **kw)
        return lib.verify_windows(*a.values(), None)

    assert call(p=None) == -1
    assert call(u=None) == -1
    assert call(tok=None) == -1
    assert call(q=None) == -1                  # drafts are drawn from q
    assert call(ud=None) == -1
    assert call(pi=None) == -1                 # every distribution output is required
    assert call(ql=None) == -1
    assert call(drafts=None) == -1
    # without drafts the q side may be NULL (the shape is still checked first)
    assert call(k=0, q=None, ud=None, drafts=None, qi=None, qp=None, ql=None, V=63) == -2
    assert call(B=0) == -2
    assert call(k=16) == -2                    # at most 15 drafts
    assert call(k=-1) == -2
    assert call(V=63) == -2                    # the pool needs 64 candidates
    assert call(V=4097) == -2                  # one top-K chunk per row
    assert call(ldp=4095) == -2
    assert call(ldq=4095) == -2
    assert call(T=float("nan")) == -3
    assert call(T=float("inf")) == -3
    assert call(top_p=float("nan")) == -3


def test_tree_attention_split_plan():
    """The workspace holds (splits x KV heads x queries) partial results of
    130 floats, so its size shows the plan: about 256 / KV heads context
    splits of whole 64-key sub-blocks (one workgroup per CU), plus the
    scratch slots' split."""
    lib = vs.library()
    per = lambda Hkv, M: Hkv * M * 130 * 4
    # 3 x 8 tree, 32/8 heads (100 queries per KV head), context 2080: 33
    # sub-blocks in 17 splits of two, plus the slots
    assert lib.tree_attention_rows_workspace_bytes(25, 32, 8, 2080) == 18 * per(8, 100)
    # 8000 positions (125 sub-blocks): 32 splits of four
    assert lib.tree_attention_rows_workspace_bytes(9, 32, 8, 8000) == 33 * per(8, 36)
    # 16 KV heads, 2000 positions: 16 splits of two
    assert lib.tree_attention_rows_workspace_bytes(9, 32, 16, 2000) == 17 * per(16, 18)
    # one KV head, 40000 positions (625 sub-blocks): 209 splits of three
    assert lib.tree_attention_rows_workspace_bytes(5, 4, 1, 40000) == 210 * per(1, 20)
    # no context: the slots' split alone
    assert lib.tree_attention_rows_workspace_bytes(25, 32, 8, 0) == 1 * per(8, 100)


def test_verify_window_rejects_before_launch():
    """The fused acceptance stage checks shapes, parameters and the workspace
    on the host (its workspace is topk_rows' at K = 64)."""
    lib = vs.library()
    V = 151936
    assert lib.verify_window_workspace_bytes(4, V) == lib.topk_rows_workspace_bytes(4, V, 64)
    assert lib.verify_window_workspace_bytes(4, 1024) == 0
    ws = lib.verify_window_workspace_bytes(4, V)
    base = dict(logits=FAKE, ld=V, R=4, V=V, ctx=FAKE, n_ctx=100, drafts=FAKE, window=64, rep=1.1,
                pres=1.5, freq=0.2, qi=FAKE, qv=FAKE, q_ld=8, q_m=8, q_pen=None, T=0.7, top_k=20,
                top_p=0.95, min_p=0.05, u=FAKE, pv=FAKE, pi=FAKE, di=FAKE, dp=FAKE, dl=FAKE, qdi=FAKE,
                qdp=FAKE, qdl=FAKE, tok=FAKE, n=FAKE, ws=FAKE, nws=ws)

    def call(**kw):
        a = dict(base, **kw)
        return lib.verify_window(*a.values(), None)

    assert call(logits=None) == -1
    assert call(R=0) == -2
    assert call(R=65) == -2                      # at most 64 rows
    assert call(V=63, ld=63) == -2               # the pool needs 64 entries
    assert call(ld=V - 1) == -2
    assert call(drafts=None) == -1
    assert call(window=5000) == -3
    assert call(rep=0.0) == -3
    assert call(T=float("nan")) == -3
    assert call(u=None) == -1                    # sampled needs uniforms
    assert call(qi=None) == -1                   # and the draft's candidates
    assert call(q_m=65, q_ld=65) == -2
    assert call(q_ld=7) == -2                    # q_ld < q_m
    assert call(nws=ws - 1) == -5
    assert call(ws=ctypes.c_void_p(0x100008)) == -6


def test_gemv_dispatch_rule():
    """Which (N, K, R) run the split-K kernel (exactly the calls that report a
    workspace).  The 8B-class shapes keep the choices their sweeps made; on
    the hidden-5120 shapes, whose 16-row tiles give 320 row-block
    workgroups (1.25 rounds of the 256 CUs), the fill model moves down to
    split-K at every R, o from 7 rows and gate|up from 5."""
    lib = vs.library()

    def split_k_rows(N, K):
        return [R for R in range(1, 25) if lib.verify_gemv_rows_workspace_bytes(N, K, R) > 0]

    above16 = list(range(17, 25))
    assert split_k_rows(6144, 4096) == above16          # q|k|v
    assert split_k_rows(24576, 4096) == above16         # gate|up
    assert split_k_rows(4096, 12288) == list(range(9, 25))   # down: long rows
    assert split_k_rows(4096, 4096) == []               # o: under 48 MB
    assert split_k_rows(151936, 4096) == []             # LM head
    assert split_k_rows(5120, 17408) == list(range(1, 25))
    assert split_k_rows(5120, 5120) == list(range(7, 25))
    assert split_k_rows(34816, 5120) == list(range(5, 25))
    assert split_k_rows(2560, 9728) == list(range(9, 25))
    assert split_k_rows(6144, 2560) == [] and split_k_rows(151936, 2560) == []
