"""Python binding of libverify_sampling.so (the speculative-decoding verify step).

Thin ctypes marshalling over the C ABI declared in include/verify_sampling.h:
each function checks dtype, device, contiguity and shapes of the torch
tensors it is given, passes their device pointers and the current HIP
stream, and raises VerifySamplingError on a non-zero status.  All the work
runs in the library's HIP kernels; there is no fallback path.  If the
library has not been built, importing this package succeeds but every call
raises.

Build the library with ``python -m verify_sampling_amd.build``.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libverify_sampling.so")

__all__ = [
    "VerifySamplingError",
    "library",
    "verify_gemv_rows",
    "verify_gemv_rows_workspace_bytes",
    "penalize_rows",
    "penalize_tree_rows",
    "topk_rows",
    "topk_rows_workspace_bytes",
    "topk_rows_noalloc",
    "sample_policy_rows",
    "spec_accept_rows",
    "verify_window",
    "verify_window_workspace_bytes",
    "verify_tree_window",
    "verify_windows",
    "choose_depth",
    "lookup_tree",
    "tree_attention_rows",
    "tree_attention_rows_workspace_bytes",
    "tree_commit_kv",
    "ACCEPT_SAMPLED",
    "ACCEPT_GREEDY",
    "ACCEPT_GREEDY_TREE",
    "ACCEPT_POINT_MASS",
    "ACCEPT_NAIVE",
    "ACCEPT_NAIVE_TREE",
    "POOL",
    "MAX_ROWS",
    "EXPORTED_SYMBOLS",
]

(ACCEPT_SAMPLED, ACCEPT_GREEDY, ACCEPT_GREEDY_TREE, ACCEPT_POINT_MASS, ACCEPT_NAIVE,
 ACCEPT_NAIVE_TREE) = 0, 1, 2, 3, 4, 5
POOL = 64
MAX_ROWS = 24

EXPORTED_SYMBOLS = (
    "vs_abi_version",
    "vs_status_string",
    "vs_last_error_detail",
    "verify_gemv_rows_workspace_bytes",
    "verify_gemv_rows",
    "penalize_rows",
    "penalize_tree_rows",
    "topk_rows_workspace_bytes",
    "topk_rows",
    "topk_rows_noalloc_max_scratch_bytes",
    "topk_rows_noalloc",
    "sample_policy_rows",
    "spec_accept_rows",
    "verify_window_workspace_bytes",
    "verify_window",
    "verify_tree_window",
    "verify_windows",
    "tree_attention_rows_workspace_bytes",
    "tree_attention_rows",
    "tree_commit_kv",
    "vs_choose_depth",
    "vs_lookup_tree",
)


class VerifySamplingError(RuntimeError):
    pass


_lib = None
P = ctypes.c_void_p
I32 = ctypes.c_int
I64 = ctypes.c_int64
F32 = ctypes.c_float
SZ = ctypes.c_size_t

_SIGNATURES = {
    "vs_abi_version": ([], I32),
    "vs_status_string": ([I32], ctypes.c_char_p),
    "vs_last_error_detail": ([], ctypes.c_char_p),
    "verify_gemv_rows_workspace_bytes": ([I32, I32, I32], SZ),
    "verify_gemv_rows": ([P, I64, I32, I32, P, I64, I32, P, I64, P, SZ, P], I32),
    "penalize_rows": ([P, P, I64, I32, I32, I32, P, I32, P, I32, I32, F32, F32, F32, P], I32),
    "penalize_tree_rows": ([P, P, I64, I32, I32, P, I32, P, P, I32, I32, F32, F32, F32, P], I32),
    "topk_rows_workspace_bytes": ([I32, I32, I32], SZ),
    "topk_rows": ([P, I64, I32, I32, I32, P, P, I64, P, SZ, P], I32),
    "topk_rows_noalloc_max_scratch_bytes": ([], SZ),
    "topk_rows_noalloc": ([P, I64, I32, I32, I32, P, P, I64, P], I32),
    "sample_policy_rows": ([P, P, I64, I32, I32, F32, I32, F32, F32, P, P, P, I64, P, P, P], I32),
    "spec_accept_rows": ([I32, I32, I32, P, P, P, I32, I64, P, P, P, I32, I64, P, P, P, P, P, P],
                         I32),
    "verify_window_workspace_bytes": ([I32, I32], SZ),
    "verify_window": ([P, I64, I32, I32, P, I32, P, I32, F32, F32, F32, P, P, I64, I32, P, F32, I32, F32,
                       F32, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P], I32),
    "verify_tree_window": ([P, I64, I32, I32, P, I32, P, P, I32, F32, F32, F32, F32, I32, F32, F32, P, P, P,
                            P, P, P, P, P, P, SZ, P], I32),
    "verify_windows": ([P, I64, P, I64, I32, I32, I32, F32, I32, F32, F32, P, P, P, P, P, P, P, P, P, P, P,
                        P], I32),
    "tree_attention_rows_workspace_bytes": ([I32, I32, I32, I32], SZ),
    "tree_attention_rows": ([P, I32, I32, I32, P, P, I64, I32, P, P, I32, P, I32, F32, P, P, SZ, P], I32),
    "tree_commit_kv": ([P, P, I64, I32, P, P, I32, P, I32, I32, I32, P], I32),
    "vs_choose_depth": ([P, I32, P, P], I32),
    "vs_lookup_tree": ([P, I32, I32, I32, I32, I32, P, P], I32),
}


def library(path: str | None = None):
    """Loads (once) and returns the ctypes handle of the built library."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise VerifySamplingError(
            f"{path} is missing: build it with `python -m verify_sampling_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != 0:
        lib = library()
        msg = lib.vs_status_string(status).decode()
        detail = lib.vs_last_error_detail().decode() if status == -7 else ""
        raise VerifySamplingError(f"{what}: {msg} ({status}) {detail}".rstrip())


def _stream(stream=None) -> int:
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t, dtype, name, allow_none=False, device=None):
    """Device pointer of t after checking its type, dtype and device."""
    import torch

    if t is None:
        if allow_none:
            return None
        raise VerifySamplingError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise VerifySamplingError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise VerifySamplingError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise VerifySamplingError(f"{name} must be on the GPU")
    if device is not None and t.device != device:
        raise VerifySamplingError(f"{name} is on {t.device}, the call's tensors on {device}")
    return t.data_ptr()


def _ld(t, name):
    """Leading dimension (in elements) of a 2-D row-major tensor with unit column stride."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise VerifySamplingError(f"{name} must be 2-D with contiguous rows")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


def _mat(t, name, rows, cols, dtype, device, *, exact_rows=True):
    """Checks a 2-D row-major operand of at least rows x cols (exactly `rows`
    rows unless exact_rows is False) and returns (pointer, leading dimension)."""
    ptr = _ptr(t, dtype, name, device=device)
    ld = _ld(t, name)
    r, c = t.shape
    if (r != rows if exact_rows else r < rows) or c < cols:
        want = f"[{rows}]" if exact_rows else f"[>= {rows}]"
        raise VerifySamplingError(f"{name} must be {want}[>= {cols}], got {list(t.shape)}")
    return ptr, ld


def _vec(t, name, n, dtype, device, allow_none=False):
    """Checks a contiguous tensor of at least n elements; returns its pointer."""
    if t is None:
        if allow_none:
            return None
        raise VerifySamplingError(f"{name} is required")
    ptr = _ptr(t, dtype, name, device=device)
    if not t.is_contiguous():
        raise VerifySamplingError(f"{name} must be contiguous")
    if t.numel() < n:
        raise VerifySamplingError(f"{name} has {t.numel()} elements, needs {n}")
    return ptr


def _ids1d(t, name, dtype, device):
    """(pointer or None, length) of an optional 1-D contiguous id array."""
    if t is None or t.numel() == 0:
        if t is not None:
            _ptr(t, dtype, name, device=device)
        return None, 0
    if t.dim() != 1:
        raise VerifySamplingError(f"{name} must be 1-D")
    return _vec(t, name, t.numel(), dtype, device), int(t.numel())


def _workspace(t, name, device):
    """(pointer, bytes) of an optional uint8 workspace (1-D, contiguous)."""
    if t is None:
        return None, 0
    ptr = _vec(t, name, 0, _torch().uint8, device)
    return ptr, int(t.numel())


def _torch():
    import torch

    return torch


def verify_gemv_rows_workspace_bytes(N: int, K: int, R: int) -> int:
    """Bytes of the optional workspace that lets verify_gemv_rows take its fastest path."""
    return int(library().verify_gemv_rows_workspace_bytes(N, K, R))


def verify_gemv_rows(W, X, Y=None, stream=None, workspace="auto"):
    """Y[R][N] = X[R][K] @ W[N][K]^T with bf16 W, fp32 X and fp32 accumulation.

    W: torch.bfloat16 [N][K] (or int16/uint16 holding bf16 bits); X: float32
    [R][K]; Y: optional float32 [R][N] output.  workspace: "auto" allocates
    the optional workspace when the call can use one, None runs without it
    (same bits), or a uint8 device tensor.  Returns Y.
    """
    import torch

    if not isinstance(W, torch.Tensor) or not isinstance(X, torch.Tensor):
        raise VerifySamplingError("W and X must be torch tensors")
    if W.dtype in (torch.int16, torch.uint16):
        W = W.view(torch.bfloat16)
    if W.dim() != 2 or X.dim() != 2:
        raise VerifySamplingError("W and X must be 2-D")
    N, K = W.shape
    R = X.shape[0]
    dev = X.device
    w_ptr, ldw = _mat(W, "W", N, K, torch.bfloat16, dev)
    x_ptr, ldx = _mat(X, "X", R, K, torch.float32, dev)
    if X.shape[1] != K:
        raise VerifySamplingError(f"X must be [R][{K}], got {list(X.shape)}")
    if Y is None:
        Y = torch.empty((R, N), dtype=torch.float32, device=dev)
    y_ptr, ldy = _mat(Y, "Y", R, N, torch.float32, dev)
    if Y.shape[1] != N:
        raise VerifySamplingError(f"Y must be [{R}][{N}], got {list(Y.shape)}")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise VerifySamplingError('workspace must be "auto", None or a uint8 tensor')
        nbytes = verify_gemv_rows_workspace_bytes(N, K, R)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    ws_ptr, ws_bytes = _workspace(workspace, "workspace", dev)
    st = library().verify_gemv_rows(w_ptr, ldw, N, K, x_ptr, ldx, R, y_ptr, ldy, ws_ptr, ws_bytes,
                                    _stream(stream))
    _check(st, "verify_gemv_rows")
    return Y


def _logit_rows(logits, ids, vocab):
    """(logits ptr, ids ptr or None, ld, rows, width, vocab) of a dense or sparse call."""
    import torch

    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise VerifySamplingError("logits must be a 2-D torch tensor")
    rows, width = logits.shape
    dev = logits.device
    l_ptr, ld = _mat(logits, "logits", rows, width, torch.float32, dev)
    i_ptr = None
    if ids is None:
        vocab = width if vocab is None else vocab
    else:
        if vocab is None:
            raise VerifySamplingError("vocab is required in sparse mode")
        i_ptr, _ = _mat(ids, "ids", rows, width, torch.int32, dev)
        if tuple(ids.shape) != (rows, width) or ids.stride() != logits.stride():
            raise VerifySamplingError("ids must match logits in shape and strides")
    return l_ptr, i_ptr, ld, rows, width, int(vocab)


def penalize_rows(logits, ctx, drafts, *, window, repeat, presence, frequency, vocab=None,
                  ids=None, stream=None):
    """In-place penalties: row i of `logits` uses H_i = last `window` of ctx || drafts[:i].

    Dense: logits float32 [rows][V] (vocab defaults to V).  Sparse: `ids`
    int32 [rows][M] and logits [rows][M] candidate slots, `vocab` required.
    ctx, drafts: int32 1-D contiguous device tensors (may be empty or None).
    """
    import torch

    l_ptr, i_ptr, ld, rows, width, vocab = _logit_rows(logits, ids, vocab)
    dev = logits.device
    c_ptr, n_ctx = _ids1d(ctx, "ctx", torch.int32, dev)
    d_ptr, n_d = _ids1d(drafts, "drafts", torch.int32, dev)
    st = library().penalize_rows(l_ptr, i_ptr, ld, rows, width, vocab, c_ptr, n_ctx, d_ptr, n_d,
                                 int(window), float(repeat), float(presence), float(frequency),
                                 _stream(stream))
    _check(st, "penalize_rows")
    return logits


def penalize_tree_rows(logits, ctx, tokens, parent, *, window, repeat, presence, frequency,
                       vocab=None, ids=None, stream=None):
    """In-place penalties on the n_nodes + 1 rows of a token tree.

    Row 0 (root) uses the last `window` of ctx; row 1 + j (node j) the last
    `window` of ctx || the path from the root down to node j.  tokens,
    parent: int32 [n_nodes] 1-D contiguous device tensors (parent -1 =
    root).  Dense or sparse as penalize_rows.
    """
    import torch

    l_ptr, i_ptr, ld, rows, width, vocab = _logit_rows(logits, ids, vocab)
    dev = logits.device
    t_ptr, n_nodes = _ids1d(tokens, "tokens", torch.int32, dev)
    p_ptr, n_par = _ids1d(parent, "parent", torch.int32, dev)
    if n_par != n_nodes:
        raise VerifySamplingError(f"parent has {n_par} entries, tokens {n_nodes}")
    if rows != n_nodes + 1:
        raise VerifySamplingError(f"a tree of {n_nodes} nodes has {n_nodes + 1} rows, got {rows}")
    c_ptr, n_ctx = _ids1d(ctx, "ctx", torch.int32, dev)
    st = library().penalize_tree_rows(l_ptr, i_ptr, ld, width, vocab, c_ptr, n_ctx, t_ptr, p_ptr,
                                      n_nodes, int(window), float(repeat), float(presence),
                                      float(frequency), _stream(stream))
    _check(st, "penalize_tree_rows")
    return logits


def topk_rows_workspace_bytes(rows: int, V: int, K: int) -> int:
    return int(library().topk_rows_workspace_bytes(rows, V, K))


def topk_rows(X, K, out_vals=None, out_idx=None, workspace=None, stream=None):
    """Per-row top-K of float32 X [rows][V] in pool order -> (vals [rows][K], idx int32).

    out_vals / out_idx: optional [rows][>= K] outputs with equal strides;
    workspace: optional uint8 device tensor (allocated here when needed and
    not given).
    """
    import torch

    if not isinstance(X, torch.Tensor) or X.dim() != 2:
        raise VerifySamplingError("X must be a 2-D torch tensor")
    rows, V = X.shape
    K = int(K)
    dev = X.device
    x_ptr, ldx = _mat(X, "X", rows, V, torch.float32, dev)
    if out_vals is None:
        out_vals = torch.empty((rows, K), dtype=torch.float32, device=dev)
    if out_idx is None:
        out_idx = torch.empty((rows, K), dtype=torch.int32, device=dev)
    v_ptr, ld_out = _mat(out_vals, "out_vals", rows, K, torch.float32, dev)
    o_ptr, _ = _mat(out_idx, "out_idx", rows, K, torch.int32, dev)
    if out_vals.stride() != out_idx.stride() or out_vals.shape != out_idx.shape:
        raise VerifySamplingError("out_vals and out_idx must share shape and strides")
    need = topk_rows_workspace_bytes(rows, V, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _workspace(workspace, "workspace", dev)
    st = library().topk_rows(x_ptr, ldx, rows, V, K, v_ptr, o_ptr, ld_out, ws_ptr, ws_bytes,
                             _stream(stream))
    _check(st, "topk_rows")
    return out_vals, out_idx


def topk_rows_noalloc(X, K, out_vals=None, out_idx=None, stream=None):
    """topk_rows without a workspace: the library's fixed per-GPU scratch
    area holds the per-chunk candidates (no allocation in the library; pass
    out_vals and out_idx to allocate nothing here either).  Calls that may
    overlap on one GPU share that area and must be serialised."""
    import torch

    if not isinstance(X, torch.Tensor) or X.dim() != 2:
        raise VerifySamplingError("X must be a 2-D torch tensor")
    rows, V = X.shape
    K = int(K)
    dev = X.device
    x_ptr, ldx = _mat(X, "X", rows, V, torch.float32, dev)
    if out_vals is None:
        out_vals = torch.empty((rows, K), dtype=torch.float32, device=dev)
    if out_idx is None:
        out_idx = torch.empty((rows, K), dtype=torch.int32, device=dev)
    v_ptr, ld_out = _mat(out_vals, "out_vals", rows, K, torch.float32, dev)
    o_ptr, _ = _mat(out_idx, "out_idx", rows, K, torch.int32, dev)
    if out_vals.stride() != out_idx.stride() or out_vals.shape != out_idx.shape:
        raise VerifySamplingError("out_vals and out_idx must share shape and strides")
    st = library().topk_rows_noalloc(x_ptr, ldx, rows, V, K, v_ptr, o_ptr, ld_out, _stream(stream))
    _check(st, "topk_rows_noalloc")
    return out_vals, out_idx


def sample_policy_rows(vals, ids, *, temperature, top_k, top_p, min_p, u=None, out=None,
                       stream=None):
    """Policy over candidate rows vals float32 [rows][M], ids int32 [rows][M] (M <= 64).

    Returns (dist_ids int32 [rows][M], dist_probs float32 [rows][M],
    dist_len int32 [rows], drawn int32 [rows] or None).  u: optional float32
    [rows] uniforms (then drawn is returned).  out: optional preallocated
    (dist_ids, dist_probs, dist_len, drawn) with drawn None when u is None.
    """
    import torch

    if not isinstance(vals, torch.Tensor) or vals.dim() != 2:
        raise VerifySamplingError("vals must be a 2-D torch tensor")
    rows, M = vals.shape
    dev = vals.device
    v_ptr, ld = _mat(vals, "vals", rows, M, torch.float32, dev)
    i_ptr, _ = _mat(ids, "ids", rows, M, torch.int32, dev)
    if tuple(ids.shape) != (rows, M) or ids.stride() != vals.stride():
        raise VerifySamplingError("ids must match vals in shape and strides")
    if out is None:
        out = (torch.empty((rows, M), dtype=torch.int32, device=dev),
               torch.empty((rows, M), dtype=torch.float32, device=dev),
               torch.empty((rows,), dtype=torch.int32, device=dev),
               torch.empty((rows,), dtype=torch.int32, device=dev) if u is not None else None)
    d_ids, d_probs, d_len, drawn = out
    di_ptr, ld_dist = _mat(d_ids, "dist_ids", rows, M, torch.int32, dev)
    dp_ptr, _ = _mat(d_probs, "dist_probs", rows, M, torch.float32, dev)
    if d_ids.stride() != d_probs.stride() or d_ids.shape != d_probs.shape:
        raise VerifySamplingError("dist_ids and dist_probs must share shape and strides")
    dl_ptr = _vec(d_len, "dist_len", rows, torch.int32, dev)
    if (u is None) != (drawn is None):
        raise VerifySamplingError("u and drawn must be given together")
    u_ptr = _vec(u, "u", rows, torch.float32, dev, allow_none=True)
    dr_ptr = _vec(drawn, "drawn", rows, torch.int32, dev, allow_none=True)
    st = library().sample_policy_rows(v_ptr, i_ptr, ld, rows, M, float(temperature), int(top_k),
                                      float(top_p), float(min_p), di_ptr, dp_ptr, dl_ptr, ld_dist,
                                      u_ptr, dr_ptr, _stream(stream))
    _check(st, "sample_policy_rows")
    return d_ids, d_probs, d_len, drawn


def verify_windows(p_logits, q_logits, k, *, temperature, top_k, top_p, min_p, u_draft, u,
                   drafts=None, p_dist=None, q_dist=None, out=None, stream=None):
    """The sampled acceptance stage of B windows in one launch.

    p_logits float32 [B * (k + 1)][V] (window b's target row i is row
    b * (k + 1) + i), q_logits float32 [B * k][V] (draft row i of window b is
    row b * k + i; None when k = 0), 64 <= V <= 4096, 0 <= k <= 15.
    u_draft float32 [B * k] draws the drafts from q; u float32 [B][k + 1][2]
    as for spec_accept_rows.  Outputs, allocated here when not given:
    drafts int32 [B * k]; p_dist (ids int32, probs float32 [B * (k + 1)][64],
    len int32 [B * (k + 1)]); q_dist likewise [B * k]; out (tokens int32
    [B][k + 1], n int32 [B]).  Returns (tokens, n).
    """
    import torch

    if not isinstance(p_logits, torch.Tensor) or p_logits.dim() != 2:
        raise VerifySamplingError("p_logits must be a 2-D torch tensor")
    k = int(k)
    if k < 0 or k > 15:
        raise VerifySamplingError(f"k must be in [0, 15], got {k}")
    rows_p, V = p_logits.shape
    if rows_p % (k + 1) != 0:
        raise VerifySamplingError(f"p_logits rows ({rows_p}) must be a multiple of k + 1 = {k + 1}")
    B = rows_p // (k + 1)
    dev = p_logits.device
    p_ptr, ldp = _mat(p_logits, "p_logits", B * (k + 1), V, torch.float32, dev)
    if p_logits.shape[1] != V:
        raise VerifySamplingError("p_logits must hold exactly V columns")
    q_ptr, ldq = None, V
    if k > 0:
        if q_logits is None:
            raise VerifySamplingError("q_logits is required when k > 0")
        q_ptr, ldq = _mat(q_logits, "q_logits", B * k, V, torch.float32, dev)
        if q_logits.shape[1] != V:
            raise VerifySamplingError("q_logits must have as many columns as p_logits")
    ud_ptr = _vec(u_draft, "u_draft", B * k, torch.float32, dev, allow_none=k == 0)
    u_ptr = _vec(u, "u", B * (k + 1) * 2, torch.float32, dev)
    if drafts is None:
        drafts = torch.empty((B * k,), dtype=torch.int32, device=dev)
    dr_ptr = _vec(drafts, "drafts", B * k, torch.int32, dev) if k > 0 else None

    # outputs the caller leaves out are allocated here and held until the
    # launch is enqueued (a freed block could be handed to the next output)
    if p_dist is None:
        p_dist = (torch.empty((B * (k + 1), POOL), dtype=torch.int32, device=dev),
                  torch.empty((B * (k + 1), POOL), dtype=torch.float32, device=dev),
                  torch.empty((B * (k + 1),), dtype=torch.int32, device=dev))
    if q_dist is None and k > 0:
        q_dist = (torch.empty((B * k, POOL), dtype=torch.int32, device=dev),
                  torch.empty((B * k, POOL), dtype=torch.float32, device=dev),
                  torch.empty((B * k,), dtype=torch.int32, device=dev))

    def dist(d, name, rows):
        if rows == 0:
            return None, None, None
        ids, probs, length = d
        i_ptr = _vec(ids, f"{name}_ids", rows * POOL, torch.int32, dev)
        p_ptr_ = _vec(probs, f"{name}_probs", rows * POOL, torch.float32, dev)
        l_ptr = _vec(length, f"{name}_len", rows, torch.int32, dev)
        return i_ptr, p_ptr_, l_ptr

    pi, pp, pl = dist(p_dist, "p", B * (k + 1))
    qi, qp, ql = dist(q_dist, "q", B * k)
    if out is None:
        out = (torch.empty((B, k + 1), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    tokens, n = out
    t_ptr = _vec(tokens, "out_tokens", B * (k + 1), torch.int32, dev)
    n_ptr = _vec(n, "out_n", B, torch.int32, dev)
    st = library().verify_windows(p_ptr, ldp, q_ptr, ldq, B, k, V, float(temperature), int(top_k),
                                  float(top_p), float(min_p), ud_ptr, u_ptr, dr_ptr, pi, pp, pl,
                                  qi, qp, ql, t_ptr, n_ptr, _stream(stream))
    _check(st, "verify_windows")
    return tokens, n


_TREE_MODES = (ACCEPT_GREEDY_TREE, ACCEPT_NAIVE_TREE)
_UNIFORM_MODES = (ACCEPT_SAMPLED, ACCEPT_POINT_MASS, ACCEPT_NAIVE, ACCEPT_NAIVE_TREE)
_GREEDY_MODES = (ACCEPT_GREEDY, ACCEPT_GREEDY_TREE)


def _dist_rows(dist, name, rows, dev, need_probs):
    """Pointers (ids, probs, len) and the row width of one side's sparse rows.

    ids [>= rows][w] with rows of exactly w entries (the kernel reads up to
    w per row), probs of the same shape and strides, len [>= rows]."""
    import torch

    ids, probs, length = dist
    i_ptr, ld = _mat(ids, f"{name}_ids", rows, 1, torch.int32, dev, exact_rows=False)
    w = ids.shape[1]
    if ids.shape[0] > 1 and ld != w:
        raise VerifySamplingError(f"{name}_ids rows must be dense (stride {w}), got stride {ld}")
    if w > POOL:
        raise VerifySamplingError(f"{name}_ids rows hold at most {POOL} entries, got {w}")
    if need_probs and (probs is None or length is None):
        raise VerifySamplingError(f"{name}_probs and {name}_len are required in this mode")
    p_ptr = None
    if probs is not None:
        p_ptr, _ = _mat(probs, f"{name}_probs", ids.shape[0], w, torch.float32, dev)
        if probs.shape != ids.shape or probs.stride() != ids.stride():
            raise VerifySamplingError(f"{name}_probs must match {name}_ids in shape and strides")
    l_ptr = _vec(length, f"{name}_len", rows, torch.int32, dev, allow_none=True)
    return i_ptr, p_ptr, l_ptr, w


def spec_accept_rows(mode, drafts, p, q=None, *, u=None, parent=None, p_win_stride=None,
                     q_win_stride=None, out=None, stream=None):
    """Accept drafts of B windows.

    drafts: int32 [B][k].  p = (ids int32 [P][w], probs float32 [P][w] or
    None, len int32 [P] or None) with window b's row i at row
    b * p_win_stride + i (default stride k + 1); q likewise with k rows per
    window (default stride k; sampled mode only).  u: float32 [B][k+1][2]
    (sampled, point-mass and naive modes); parent: int32 [B][k] (tree
    modes).  Returns (tokens int32 [B][k+1], n_emitted int32 [B]).
    """
    import torch

    mode = int(mode)
    if not isinstance(drafts, torch.Tensor) or drafts.dim() != 2:
        raise VerifySamplingError("drafts must be a 2-D torch tensor [B][k]")
    B, k = drafts.shape
    dev = drafts.device
    d_ptr = _vec(drafts, "drafts", B * k, torch.int32, dev)
    p_ws = k + 1 if p_win_stride is None else int(p_win_stride)
    q_ws = k if q_win_stride is None else int(q_win_stride)
    if p_ws < 0 or q_ws < 0:
        raise VerifySamplingError("window strides must be >= 0")
    p_rows = (B - 1) * p_ws + k + 1
    pi_ptr, pp_ptr, pl_ptr, p_ld = _dist_rows(p, "p", p_rows, dev, mode not in _GREEDY_MODES)
    q_ptrs, q_ld = (None, None, None), 1
    if mode == ACCEPT_SAMPLED and k > 0:
        if q is None:
            raise VerifySamplingError("q is required in sampled mode")
        *q_ptrs, q_ld = _dist_rows(q, "q", (B - 1) * q_ws + k, dev, True)
    u_ptr = None
    if mode in _UNIFORM_MODES:
        if u is None:
            raise VerifySamplingError("u is required in this mode")
        u_ptr = _vec(u, "u", B * (k + 1) * 2, torch.float32, dev)
    par_ptr = None
    if mode in _TREE_MODES:
        if parent is None:
            raise VerifySamplingError("parent is required in the tree modes")
        par_ptr = _vec(parent, "parent", B * k, torch.int32, dev)
    if out is None:
        out = (torch.empty((B, k + 1), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    tokens, n_emitted = out
    t_ptr = _vec(tokens, "tokens", B * (k + 1), torch.int32, dev)
    n_ptr = _vec(n_emitted, "n_emitted", B, torch.int32, dev)
    st = library().spec_accept_rows(mode, B, k, pi_ptr, pp_ptr, pl_ptr, p_ld, p_ws, q_ptrs[0],
                                    q_ptrs[1], q_ptrs[2], q_ld, q_ws, d_ptr, par_ptr, u_ptr, t_ptr,
                                    n_ptr, _stream(stream))
    _check(st, "spec_accept_rows")
    return tokens, n_emitted


def verify_window_workspace_bytes(R: int, V: int) -> int:
    return int(library().verify_window_workspace_bytes(R, V))


def verify_window(logits, ctx, drafts, *, window, repeat, presence, frequency, temperature, top_k,
                  top_p, min_p, q_ids=None, q_vals=None, u=None, out=None, workspace=None,
                  stream=None):
    """The acceptance stage of one chain window in two launches.

    logits float32 [R][V] (penalised in place); ctx int32 [n] and drafts
    int32 [R - 1] 1-D device tensors.  Sampled (temperature > 0) also needs
    q_ids int32 / q_vals float32 [R - 1][M] (equal strides; not changed) and
    u float32 [R][2].  Returns a dict: tokens int32 [R] (-1 past the count),
    n int32 [1], pool_vals / pool_ids [R][64], p = (ids, probs, len) of the
    target rows, q = (ids, probs, len) and q_pen (the penalised candidates)
    in sampled mode, else None.  out: an optional dict of the same outputs,
    preallocated (q entries [R - 1][ld of q_vals]).
    """
    import torch

    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise VerifySamplingError("logits must be a 2-D torch tensor [R][V]")
    R, V = logits.shape
    k = R - 1
    dev = logits.device
    l_ptr, ld = _mat(logits, "logits", R, V, torch.float32, dev)
    c_ptr, n_ctx = _ids1d(ctx, "ctx", torch.int32, dev)
    d_ptr, n_d = _ids1d(drafts, "drafts", torch.int32, dev)
    if n_d != k:
        raise VerifySamplingError(f"{R} rows verify {k} drafts, got {n_d}")
    sampled = float(temperature) > 0
    qi_ptr = qv_ptr = u_ptr = None
    q_ld, q_m = 1, 1
    if sampled:
        u_ptr = _vec(u, "u", R * 2, torch.float32, dev)
        if k > 0:
            qv_ptr, q_ld = _mat(q_vals, "q_vals", k, 1, torch.float32, dev)
            q_m = q_vals.shape[1]
            qi_ptr, _ = _mat(q_ids, "q_ids", k, q_m, torch.int32, dev)
            if tuple(q_ids.shape) != tuple(q_vals.shape) or q_ids.stride() != q_vals.stride():
                raise VerifySamplingError("q_ids must match q_vals in shape and strides")
            if q_m > POOL:
                raise VerifySamplingError(f"q rows hold at most {POOL} candidates, got {q_m}")
    if out is None:
        out = dict(tokens=torch.empty((R,), dtype=torch.int32, device=dev),
                   n=torch.empty((1,), dtype=torch.int32, device=dev),
                   pool_vals=torch.empty((R, POOL), dtype=torch.float32, device=dev),
                   pool_ids=torch.empty((R, POOL), dtype=torch.int32, device=dev),
                   p=(torch.empty((R, POOL), dtype=torch.int32, device=dev),
                      torch.empty((R, POOL), dtype=torch.float32, device=dev),
                      torch.empty((R,), dtype=torch.int32, device=dev)),
                   q=None, q_pen=None)
        if sampled and k > 0:
            out["q"] = (torch.empty((k, q_ld), dtype=torch.int32, device=dev),
                        torch.empty((k, q_ld), dtype=torch.float32, device=dev),
                        torch.empty((k,), dtype=torch.int32, device=dev))
            out["q_pen"] = torch.empty((k, q_ld), dtype=torch.float32, device=dev)

    def dense(t, name, rows, cols, dtype):
        ptr = _vec(t, name, rows * cols, dtype, dev)
        if tuple(t.shape) != (rows, cols):
            raise VerifySamplingError(f"{name} must be [{rows}][{cols}], got {list(t.shape)}")
        return ptr

    t_ptr = _vec(out["tokens"], "tokens", R, torch.int32, dev)
    n_ptr = _vec(out["n"], "n", 1, torch.int32, dev)
    pv_ptr = dense(out["pool_vals"], "pool_vals", R, POOL, torch.float32)
    pi_ptr = dense(out["pool_ids"], "pool_ids", R, POOL, torch.int32)
    p_ids, p_probs, p_len = out["p"]
    di_ptr = dense(p_ids, "p_ids", R, POOL, torch.int32)
    dp_ptr = dense(p_probs, "p_probs", R, POOL, torch.float32)
    dl_ptr = _vec(p_len, "p_len", R, torch.int32, dev)
    qdi_ptr = qdp_ptr = qdl_ptr = qp_ptr = None
    if sampled and k > 0:
        if out.get("q") is None:
            raise VerifySamplingError("out['q'] is required in sampled mode")
        q_d_ids, q_d_probs, q_d_len = out["q"]
        qdi_ptr = dense(q_d_ids, "q_dist_ids", k, q_ld, torch.int32)
        qdp_ptr = dense(q_d_probs, "q_dist_probs", k, q_ld, torch.float32)
        qdl_ptr = _vec(q_d_len, "q_dist_len", k, torch.int32, dev)
        if out.get("q_pen") is not None:
            qp_ptr = dense(out["q_pen"], "q_pen", k, q_ld, torch.float32)
    need = verify_window_workspace_bytes(R, V)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _workspace(workspace, "workspace", dev)
    st = library().verify_window(l_ptr, ld, R, V, c_ptr, n_ctx, d_ptr, int(window), float(repeat),
                                 float(presence), float(frequency), qi_ptr, qv_ptr, q_ld, q_m, qp_ptr,
                                 float(temperature), int(top_k), float(top_p), float(min_p), u_ptr,
                                 pv_ptr, pi_ptr, di_ptr, dp_ptr, dl_ptr, qdi_ptr, qdp_ptr, qdl_ptr,
                                 t_ptr, n_ptr, ws_ptr, ws_bytes, _stream(stream))
    _check(st, "verify_window")
    return out


def verify_tree_window(logits, ctx, tokens, parent, *, window, repeat, presence, frequency,
                       temperature, top_k, top_p, min_p, u=None, out=None, workspace=None, stream=None):
    """The acceptance stage of one token tree in two launches.

    logits float32 [R][V] (row 0 the root, row 1 + j node j; penalised in
    place, each row against the context and its own branch's path); ctx
    int32 [n] and tokens, parent int32 [R - 1] 1-D device tensors (parent
    -1 = the root).  Sampled (temperature > 0: the naive-sampling walk) also
    needs u float32 [R][2]; greedy walks the tree by the rows' argmax.
    Returns a dict: tokens int32 [R] (-1 past the count), n int32 [1],
    pool_vals / pool_ids [R][64], p = (ids, probs, len).  out: an optional
    dict of the same outputs, preallocated.
    """
    import torch

    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise VerifySamplingError("logits must be a 2-D torch tensor [R][V]")
    R, V = logits.shape
    n = R - 1
    dev = logits.device
    l_ptr, ld = _mat(logits, "logits", R, V, torch.float32, dev)
    c_ptr, n_ctx = _ids1d(ctx, "ctx", torch.int32, dev)
    t_ptr, n_tok = _ids1d(tokens, "tokens", torch.int32, dev)
    p_ptr, n_par = _ids1d(parent, "parent", torch.int32, dev)
    if n_tok != n or n_par != n:
        raise VerifySamplingError(f"a tree of {R} rows has {n} nodes: tokens {n_tok}, parent {n_par}")
    sampled = float(temperature) > 0
    u_ptr = _vec(u, "u", R * 2, torch.float32, dev) if sampled else None
    if out is None:
        out = dict(tokens=torch.empty((R,), dtype=torch.int32, device=dev),
                   n=torch.empty((1,), dtype=torch.int32, device=dev),
                   pool_vals=torch.empty((R, POOL), dtype=torch.float32, device=dev),
                   pool_ids=torch.empty((R, POOL), dtype=torch.int32, device=dev),
                   p=(torch.empty((R, POOL), dtype=torch.int32, device=dev),
                      torch.empty((R, POOL), dtype=torch.float32, device=dev),
                      torch.empty((R,), dtype=torch.int32, device=dev)))

    def dense(t, name, rows, cols, dtype):
        ptr = _vec(t, name, rows * cols, dtype, dev)
        if tuple(t.shape) != (rows, cols):
            raise VerifySamplingError(f"{name} must be [{rows}][{cols}], got {list(t.shape)}")
        return ptr

    to_ptr = _vec(out["tokens"], "tokens out", R, torch.int32, dev)
    n_ptr = _vec(out["n"], "n", 1, torch.int32, dev)
    pv_ptr = dense(out["pool_vals"], "pool_vals", R, POOL, torch.float32)
    pi_ptr = dense(out["pool_ids"], "pool_ids", R, POOL, torch.int32)
    p_ids, p_probs, p_len = out["p"]
    di_ptr = dense(p_ids, "p_ids", R, POOL, torch.int32)
    dp_ptr = dense(p_probs, "p_probs", R, POOL, torch.float32)
    dl_ptr = _vec(p_len, "p_len", R, torch.int32, dev)
    need = verify_window_workspace_bytes(R, V)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _workspace(workspace, "workspace", dev)
    st = library().verify_tree_window(l_ptr, ld, R, V, c_ptr, n_ctx, t_ptr, p_ptr, int(window), float(repeat),
                                      float(presence), float(frequency), float(temperature), int(top_k),
                                      float(top_p), float(min_p), u_ptr, pv_ptr, pi_ptr, di_ptr, dp_ptr, dl_ptr,
                                      to_ptr, n_ptr, ws_ptr, ws_bytes, _stream(stream))
    _check(st, "verify_tree_window")
    return out


def _bf16_bits(t, name, dev):
    """A bf16 (or int16/uint16 bit-pattern) 3-D contiguous tensor as its bits."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise VerifySamplingError(f"{name} must be a torch tensor")
    if t.dtype in (torch.int16, torch.uint16):
        t = t.view(torch.bfloat16)
    if t.dim() != 3:
        raise VerifySamplingError(f"{name} must be 3-D [heads][positions][D]")
    return _vec(t, name, t.numel(), torch.bfloat16, dev), t


def tree_attention_rows_workspace_bytes(R: int, Hq: int, Hkv: int, ctx_len: int) -> int:
    return int(library().tree_attention_rows_workspace_bytes(R, Hq, Hkv, ctx_len))


def tree_attention_rows(q, k_cache, v_cache, ctx_len, k_scr, v_scr, parent, *, scale, out=None,
                        workspace=None, stream=None):
    """Attention of the R rows of a token tree (root + R - 1 nodes) under the
    tree mask.  q float32 [R][Hq][D]; caches and scratch bf16 [Hkv][len][D];
    parent int32 [R - 1] (device).  Returns out float32 [R][Hq][D]."""
    import torch

    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise VerifySamplingError("q must be a 3-D torch tensor [R][Hq][D]")
    R, Hq, D = q.shape
    dev = q.device
    q_ptr = _vec(q, "q", q.numel(), torch.float32, dev)
    ks_ptr, k_scr = _bf16_bits(k_scr, "k_scr", dev)
    vs_ptr, v_scr = _bf16_bits(v_scr, "v_scr", dev)
    Hkv, scr_len, Ds = k_scr.shape
    if tuple(v_scr.shape) != (Hkv, scr_len, Ds) or Ds != D:
        raise VerifySamplingError("k_scr and v_scr must be [Hkv][scr_len][D] alike")
    kc_ptr, k_cache = _bf16_bits(k_cache, "k_cache", dev)
    vc_ptr, v_cache = _bf16_bits(v_cache, "v_cache", dev)
    if k_cache.shape[0] != Hkv or k_cache.shape[2] != D or v_cache.shape != k_cache.shape:
        raise VerifySamplingError("k_cache and v_cache must be [Hkv][cache_len][D] alike")
    cache_len = int(k_cache.shape[1])
    p_ptr = _vec(parent, "parent", R - 1, torch.int32, dev, allow_none=R == 1)
    if out is None:
        out = torch.empty((R, Hq, D), dtype=torch.float32, device=dev)
    o_ptr = _vec(out, "out", R * Hq * D, torch.float32, dev)
    need = tree_attention_rows_workspace_bytes(R, Hq, Hkv, int(ctx_len))
    if workspace is None:
        workspace = torch.empty(max(16, need), dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _workspace(workspace, "workspace", dev)
    st = library().tree_attention_rows(q_ptr, R, Hq, D, kc_ptr, vc_ptr, cache_len, int(ctx_len),
                                       ks_ptr, vs_ptr, scr_len, p_ptr, Hkv, float(scale), o_ptr,
                                       ws_ptr, ws_bytes, _stream(stream))
    _check(st, "tree_attention_rows")
    return out


def tree_commit_kv(k_cache, v_cache, ctx_len, k_scr, v_scr, path, stream=None):
    """Copies scratch slots path[i] into cache positions ctx_len + i, every KV head."""
    import torch

    dev = k_cache.device
    kc_ptr, k_cache = _bf16_bits(k_cache, "k_cache", dev)
    vc_ptr, v_cache = _bf16_bits(v_cache, "v_cache", dev)
    ks_ptr, k_scr = _bf16_bits(k_scr, "k_scr", dev)
    vs_ptr, v_scr = _bf16_bits(v_scr, "v_scr", dev)
    Hkv, cache_len, D = k_cache.shape
    if v_cache.shape != k_cache.shape or k_scr.shape[0] != Hkv or k_scr.shape[2] != D or \
            v_scr.shape != k_scr.shape:
        raise VerifySamplingError("caches [Hkv][cache_len][D] and scratch [Hkv][scr_len][D] must agree")
    n = int(path.numel()) if path is not None else 0
    pa_ptr = _vec(path, "path", n, torch.int32, dev) if n else None
    st = library().tree_commit_kv(kc_ptr, vc_ptr, cache_len, int(ctx_len), ks_ptr, vs_ptr,
                                  int(k_scr.shape[1]), pa_ptr, n, Hkv, D, _stream(stream))
    _check(st, "tree_commit_kv")


def choose_depth(alpha, cost):
    """(k*, rate): the draft depth with the most expected emitted tokens per unit cost.

    alpha: per-depth acceptance probabilities (length kmax); cost: window
    costs for 1..kmax+1 rows.  Host computation in the library.
    """
    a = (ctypes.c_double * max(1, len(alpha)))(*[float(x) for x in alpha])
    c = (ctypes.c_double * len(cost))(*[float(x) for x in cost])
    if len(cost) != len(alpha) + 1:
        raise VerifySamplingError("cost needs one entry more than alpha")
    rate = ctypes.c_double(0.0)
    k = library().vs_choose_depth(a, len(alpha), c, ctypes.byref(rate))
    if k < 0:
        _check(k, "vs_choose_depth")
    return int(k), rate.value


def lookup_tree(ctx, n: int, branches: int, depth: int, max_nodes: int = 24):
    """(tokens, parent) int32 arrays of the prompt-lookup token tree drafted from ctx.

    ctx: host sequence of token ids.  Host computation in the library.
    """
    import numpy as np

    c = np.ascontiguousarray(np.asarray(ctx, dtype=np.int32))
    tok = np.zeros(max(1, max_nodes), dtype=np.int32)
    par = np.zeros(max(1, max_nodes), dtype=np.int32)
    k = library().vs_lookup_tree(c.ctypes.data if c.size else None, int(c.size), int(n),
                                 int(branches), int(depth), int(max_nodes),
                                 tok.ctypes.data, par.ctypes.data)
    if k < 0:
        _check(k, "vs_lookup_tree")
    return tok[:k].copy(), par[:k].copy()
