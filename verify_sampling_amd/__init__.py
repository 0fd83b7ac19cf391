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
    "sample_policy_rows",
    "spec_accept_rows",
    "choose_depth",
    "lookup_tree",
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
    "sample_policy_rows",
    "spec_accept_rows",
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
    "sample_policy_rows": ([P, P, I64, I32, I32, F32, I32, F32, F32, P, P, P, I64, P, P, P], I32),
    "spec_accept_rows": ([I32, I32, I32, P, P, P, I32, I64, P, P, P, I32, I64, P, P, P, P, P, P],
                         I32),
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


def _ptr(t, dtype, name, allow_none=False):
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
    return t.data_ptr()


def _ld(t, name):
    """Leading dimension (in elements) of a 2-D row-major tensor with unit column stride."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise VerifySamplingError(f"{name} must be 2-D with contiguous rows")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


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

    if W.dtype in (torch.int16, torch.uint16):
        W = W.view(torch.bfloat16)
    if W.dtype != torch.bfloat16:
        raise VerifySamplingError("W must be bfloat16")
    N, K = W.shape
    R = X.shape[0]
    if X.dim() != 2 or X.shape[1] != K:
        raise VerifySamplingError(f"X must be [R][{K}]")
    if Y is None:
        Y = torch.empty((R, N), dtype=torch.float32, device=X.device)
    if tuple(Y.shape) != (R, N):
        raise VerifySamplingError(f"Y must be [{R}][{N}]")
    if isinstance(workspace, str):
        if workspace != "auto":
            raise VerifySamplingError('workspace must be "auto", None or a uint8 tensor')
        nbytes = verify_gemv_rows_workspace_bytes(N, K, R)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=X.device) if nbytes else None
    ws_ptr = _ptr(workspace, torch.uint8, "workspace", allow_none=True)
    ws_bytes = workspace.numel() if workspace is not None else 0
    st = library().verify_gemv_rows(_ptr(W, torch.bfloat16, "W"), _ld(W, "W"), N, K,
                                    _ptr(X, torch.float32, "X"), _ld(X, "X"), R,
                                    _ptr(Y, torch.float32, "Y"), _ld(Y, "Y"), ws_ptr, ws_bytes,
                                    _stream(stream))
    _check(st, "verify_gemv_rows")
    return Y


def penalize_rows(logits, ctx, drafts, *, window, repeat, presence, frequency, vocab=None,
                  ids=None, stream=None):
    """In-place penalties: row i of `logits` uses H_i = last `window` of ctx || drafts[:i].

    Dense: logits float32 [rows][V] (vocab defaults to V).  Sparse: `ids`
    int32 [rows][M] and logits [rows][M] candidate slots, `vocab` required.
    ctx, drafts: int32 1-D device tensors (may be empty).
    """
    import torch

    rows, width = logits.shape
    if ids is None:
        vocab = width if vocab is None else vocab
    elif vocab is None:
        raise VerifySamplingError("vocab is required in sparse mode")
    if ids is not None and (tuple(ids.shape) != (rows, width) or ids.stride() != logits.stride()):
        raise VerifySamplingError("ids must match logits in shape and strides")
    n_ctx = int(ctx.numel()) if ctx is not None else 0
    n_d = int(drafts.numel()) if drafts is not None else 0
    st = library().penalize_rows(
        _ptr(logits, torch.float32, "logits"), _ptr(ids, torch.int32, "ids", True),
        _ld(logits, "logits"), rows, width, int(vocab),
        _ptr(ctx, torch.int32, "ctx", True) if n_ctx else None, n_ctx,
        _ptr(drafts, torch.int32, "drafts", True) if n_d else None, n_d,
        int(window), float(repeat), float(presence), float(frequency), _stream(stream))
    _check(st, "penalize_rows")
    return logits


def penalize_tree_rows(logits, ctx, tokens, parent, *, window, repeat, presence, frequency,
                       vocab=None, ids=None, stream=None):
    """In-place penalties on the n_nodes + 1 rows of a token tree.

    Row 0 (root) uses the last `window` of ctx; row 1 + j (node j) the last
    `window` of ctx || the path from the root down to node j.  tokens,
    parent: int32 [n_nodes] device tensors (parent -1 = root).  Dense or
    sparse as penalize_rows.
    """
    import torch

    rows, width = logits.shape
    n_nodes = int(tokens.numel()) if tokens is not None else 0
    if rows != n_nodes + 1:
        raise VerifySamplingError(f"a tree of {n_nodes} nodes has {n_nodes + 1} rows, got {rows}")
    if ids is None:
        vocab = width if vocab is None else vocab
    elif vocab is None:
        raise VerifySamplingError("vocab is required in sparse mode")
    if ids is not None and (tuple(ids.shape) != (rows, width) or ids.stride() != logits.stride()):
        raise VerifySamplingError("ids must match logits in shape and strides")
    n_ctx = int(ctx.numel()) if ctx is not None else 0
    st = library().penalize_tree_rows(
        _ptr(logits, torch.float32, "logits"), _ptr(ids, torch.int32, "ids", True),
        _ld(logits, "logits"), width, int(vocab),
        _ptr(ctx, torch.int32, "ctx", True) if n_ctx else None, n_ctx,
        _ptr(tokens, torch.int32, "tokens", True) if n_nodes else None,
        _ptr(parent, torch.int32, "parent", True) if n_nodes else None, n_nodes,
        int(window), float(repeat), float(presence), float(frequency), _stream(stream))
    _check(st, "penalize_tree_rows")
    return logits


def topk_rows_workspace_bytes(rows: int, V: int, K: int) -> int:
    return int(library().topk_rows_workspace_bytes(rows, V, K))


def topk_rows(X, K, out_vals=None, out_idx=None, workspace=None, stream=None):
    """Per-row top-K of float32 X [rows][V] in pool order -> (vals [rows][K], idx int32)."""
    import torch

    rows, V = X.shape
    if out_vals is None:
        out_vals = torch.empty((rows, K), dtype=torch.float32, device=X.device)
    if out_idx is None:
        out_idx = torch.empty((rows, K), dtype=torch.int32, device=X.device)
    need = topk_rows_workspace_bytes(rows, V, K)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    ws_ptr = _ptr(workspace, torch.uint8, "workspace", True) if workspace is not None else None
    ws_bytes = int(workspace.numel()) if workspace is not None else 0
    if out_vals.stride() != out_idx.stride():
        raise VerifySamplingError("out_vals and out_idx must share strides")
    st = library().topk_rows(_ptr(X, torch.float32, "X"), _ld(X, "X"), rows, V, int(K),
                             _ptr(out_vals, torch.float32, "out_vals"),
                             _ptr(out_idx, torch.int32, "out_idx"), _ld(out_vals, "out_vals"),
                             ws_ptr, ws_bytes, _stream(stream))
    _check(st, "topk_rows")
    return out_vals, out_idx


def sample_policy_rows(vals, ids, *, temperature, top_k, top_p, min_p, u=None, out=None,
                       stream=None):
    """Policy over candidate rows vals float32 [rows][M], ids int32 [rows][M] (M <= 64).

    Returns (dist_ids int32 [rows][M], dist_probs float32 [rows][M],
    dist_len int32 [rows], drawn int32 [rows] or None).
    """
    import torch

    rows, M = vals.shape
    if tuple(ids.shape) != (rows, M) or ids.stride() != vals.stride():
        raise VerifySamplingError("ids must match vals in shape and strides")
    dev = vals.device
    if out is None:
        out = (torch.empty((rows, M), dtype=torch.int32, device=dev),
               torch.empty((rows, M), dtype=torch.float32, device=dev),
               torch.empty((rows,), dtype=torch.int32, device=dev),
               torch.empty((rows,), dtype=torch.int32, device=dev) if u is not None else None)
    d_ids, d_probs, d_len, drawn = out
    if d_ids.stride() != d_probs.stride():
        raise VerifySamplingError("dist_ids and dist_probs must share strides")
    st = library().sample_policy_rows(
        _ptr(vals, torch.float32, "vals"), _ptr(ids, torch.int32, "ids"), _ld(vals, "vals"), rows, M,
        float(temperature), int(top_k), float(top_p), float(min_p),
        _ptr(d_ids, torch.int32, "dist_ids"), _ptr(d_probs, torch.float32, "dist_probs"),
        _ptr(d_len, torch.int32, "dist_len"), _ld(d_ids, "dist_ids"),
        _ptr(u, torch.float32, "u", True), _ptr(drawn, torch.int32, "drawn", True),
        _stream(stream))
    _check(st, "sample_policy_rows")
    return d_ids, d_probs, d_len, drawn


def spec_accept_rows(mode, drafts, p, q=None, *, u=None, parent=None, p_win_stride=None,
                     q_win_stride=None, out=None, stream=None):
    """Accept drafts of B windows.

    drafts: int32 [B][k].  p = (ids int32 [P][p_ld], probs float32 [P][p_ld] or
    None, len int32 [P] or None) with window b's row i at row
    b * p_win_stride + i (default stride k + 1); q likewise with k rows per
    window (default stride k; sampled mode only).  u: float32 [B][k+1][2]
    (sampled, point-mass and naive modes);
    parent: int32 [B][k] (tree mode).  Returns (tokens int32 [B][k+1],
    n_emitted int32 [B]).
    """
    import torch

    B, k = drafts.shape
    p_ids, p_probs, p_len = p
    q_ids, q_probs, q_len = q if q is not None else (None, None, None)
    p_ws = k + 1 if p_win_stride is None else int(p_win_stride)
    q_ws = k if q_win_stride is None else int(q_win_stride)
    dev = drafts.device
    if out is None:
        out = (torch.empty((B, k + 1), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    tokens, n_emitted = out
    if not drafts.is_contiguous() or (u is not None and not u.is_contiguous()) or \
            (parent is not None and not parent.is_contiguous()):
        raise VerifySamplingError("drafts, u and parent must be contiguous")
    for name, t, rows_needed in (("p_ids", p_ids, (B - 1) * p_ws + k + 1),
                                 ("q_ids", q_ids, (B - 1) * q_ws + k)):
        if t is not None and t.shape[0] < rows_needed:
            raise VerifySamplingError(f"{name} has {t.shape[0]} rows, needs {rows_needed}")
    st = library().spec_accept_rows(
        int(mode), B, k,
        _ptr(p_ids, torch.int32, "p_ids"), _ptr(p_probs, torch.float32, "p_probs", True),
        _ptr(p_len, torch.int32, "p_len", True), _ld(p_ids, "p_ids"), p_ws,
        _ptr(q_ids, torch.int32, "q_ids", True), _ptr(q_probs, torch.float32, "q_probs", True),
        _ptr(q_len, torch.int32, "q_len", True), _ld(q_ids, "q_ids") if q_ids is not None else 1,
        q_ws, _ptr(drafts, torch.int32, "drafts"), _ptr(parent, torch.int32, "parent", True),
        _ptr(u, torch.float32, "u", True), _ptr(tokens, torch.int32, "tokens"),
        _ptr(n_emitted, torch.int32, "n_emitted"), _stream(stream))
    _check(st, "spec_accept_rows")
    return tokens, n_emitted


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
