"""Python binding of the MI355X lightning-indexer backward (C ABI via ctypes).

The functions here only marshal arguments: they check tensor dtypes, devices
and contiguity, allocate outputs when the caller passes none, and call the
entry points of ``libdsa_indexer_bwd.so`` with raw device pointers and the
current HIP stream.  Every step of the backward runs in the HIP kernels; there
is no fallback.  If the library is not built this module raises on first use.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "indexer_bwd_sparse",
    "indexer_bwd_sparse_noalloc",
    "IBWD_NOALLOC_SCRATCH_BYTES",
    "indexer_bwd_dense",
    "indexer_fwd_scores",
    "indexer_topk",
    "indexer_bwd_workspace_bytes",
    "indexer_bwd_strerror",
    "set_stage_hook",
    "library",
    "IBWD_OK",
    "IBWD_ERR_INVALID_ARGUMENT",
    "IBWD_ERR_UNSUPPORTED_DEVICE",
    "IBWD_ERR_HIP",
    "IBWD_FLAG_DETERMINISTIC",
    "IBWD_FLAG_ATOMIC_DK",
    "IBWD_FLAG_GLOBAL_IDS",
    "IBWD_FLAG_BF16_OUT",
    "IBWD_FLAG_DK_KEY_RANGES",
    "IBWD_FLAG_DK_SLOT_ROWS",
    "IndexerBwdError",
]

IBWD_OK = 0
IBWD_ERR_INVALID_ARGUMENT = -1
IBWD_ERR_UNSUPPORTED_DEVICE = -2
IBWD_ERR_HIP = -3
IBWD_FLAG_DETERMINISTIC = 1
IBWD_FLAG_ATOMIC_DK = 2
IBWD_FLAG_GLOBAL_IDS = 4
IBWD_FLAG_BF16_OUT = 8
IBWD_FLAG_DK_KEY_RANGES = 16
IBWD_FLAG_DK_SLOT_ROWS = 32
_DK_ROUTES = {"auto": 0, "key_ranges": IBWD_FLAG_DK_KEY_RANGES, "slot_rows": IBWD_FLAG_DK_SLOT_ROWS}
IBWD_NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa_indexer_bwd.so")
DEEPBUF_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa_indexer_bwd_deepbuf.so")
_lib = None
_HOOK_T = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_int, ctypes.c_char_p)
_hook_ref = None  # keeps the ctypes callback alive while it is installed


class IndexerBwdError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__("indexer_bwd failed (%d): %s" % (status, indexer_bwd_strerror(status)))


_loaded = {}  # path -> handle of every build loaded in this process


def library() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Route this module's calls to another build of the library while the
    block runs (a verification aid: the build with deeper buffer rings,
    DEEPBUF_LIB_PATH, must give the same bits as the library)."""
    global _lib
    prev = library()
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = prev


def _load(path: str) -> ctypes.CDLL:
    if path not in _loaded:
        if not os.path.exists(path):
            raise RuntimeError("HIP library %s is missing: run __graft_entry__.build() first" % path)
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        i64 = ctypes.c_int64
        f32 = ctypes.c_float
        lib.indexer_bwd_sparse.argtypes = [vp] * 9 + [i64] * 6 + [f32, f32, ctypes.c_uint32, vp,
                                                                  ctypes.c_size_t, vp]
        lib.indexer_bwd_sparse.restype = ctypes.c_int
        lib.indexer_bwd_sparse_noalloc.argtypes = [vp] * 9 + [i64] * 6 + [f32, f32,
                                                                          ctypes.c_uint32, vp]
        lib.indexer_bwd_sparse_noalloc.restype = ctypes.c_int
        lib.indexer_bwd_dense.argtypes = [vp] * 8 + [i64] * 6 + [f32, f32, ctypes.c_uint32, vp,
                                                                 ctypes.c_size_t, vp]
        lib.indexer_bwd_dense.restype = ctypes.c_int
        lib.indexer_fwd_scores.argtypes = [vp] * 4 + [i64] * 5 + [ctypes.c_int, i64, vp]
        lib.indexer_fwd_scores.restype = ctypes.c_int
        lib.indexer_topk.argtypes = [vp] * 3 + [i64] * 3 + [vp]
        lib.indexer_topk.restype = ctypes.c_int
        lib.indexer_bwd_workspace_bytes.argtypes = [ctypes.c_int] + [i64] * 6 + [ctypes.c_uint32]
        lib.indexer_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.indexer_bwd_strerror.argtypes = [ctypes.c_int]
        lib.indexer_bwd_strerror.restype = ctypes.c_char_p
        lib.indexer_bwd_set_stage_hook.argtypes = [_HOOK_T, ctypes.c_void_p]
        lib.indexer_bwd_set_stage_hook.restype = ctypes.c_int
        _loaded[path] = lib
    return _loaded[path]


def set_stage_hook(fn) -> None:
    """Profiling aid: fn(stage, kernel_name) runs on the host right after each
    kernel of a call is enqueued (see indexer_bwd_set_stage_hook); None removes it."""
    global _hook_ref
    if fn is None:
        library().indexer_bwd_set_stage_hook(_HOOK_T(), None)
        _hook_ref = None
        return
    cb = _HOOK_T(lambda user, stage, name: fn(int(stage), name.decode()))
    library().indexer_bwd_set_stage_hook(cb, None)
    _hook_ref = cb


def indexer_bwd_strerror(status: int) -> str:
    return library().indexer_bwd_strerror(int(status)).decode()


def indexer_bwd_workspace_bytes(dense: bool, B: int, S_q: int, S_k: int, H: int, D: int, topk: int,
                                flags: int = 0) -> int:
    return int(library().indexer_bwd_workspace_bytes(int(bool(dense)), B, S_q, S_k, H, D, topk,
                                                     flags))


def _torch():
    import torch
    return torch


def _check(t, dtype, shape, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_cuda:
        raise ValueError("%s must live on the GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(stream, device):
    """The torch stream a call runs on: the given one, else the device's current stream."""
    torch = _torch()
    return torch.cuda.current_stream(device) if stream is None else stream


def _outputs(q, k, d_q, d_w, d_k, bf16_out, stream):
    """The three outputs (allocated on `stream` when None), checked for dtype and shape."""
    torch = _torch()
    B, S_q, H, D = q.shape
    S_k = k.shape[1]
    dt = torch.bfloat16 if bf16_out else torch.float32
    shapes = ((B, S_q, H, D), (B, S_q, H), (B, S_k, D))
    with torch.cuda.stream(stream):
        out = [torch.empty(s, dtype=dt, device=q.device) if t is None else t
               for t, s in zip((d_q, d_w, d_k), shapes)]
    for t, s, name in zip(out, shapes, ("d_q", "d_w", "d_k")):
        _check(t, dt, s, name)
    return tuple(out)


def _workspace(dense, B, S_q, S_k, H, D, topk, flags, workspace, device, stream):
    """The caller's workspace, or one allocated here.  An allocated workspace
    belongs to the stream the kernels run on, so the caching allocator hands its
    memory to other work only in that stream's order, after the kernels that
    use it, even though it is released when this call returns."""
    torch = _torch()
    need = indexer_bwd_workspace_bytes(dense, B, S_q, S_k, H, D, topk, flags)
    if need == 0:
        return workspace, 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace is None:
        with torch.cuda.stream(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _flags(deterministic: bool, atomic_dk: bool, bf16_out: bool, dk_route: str = "auto") -> int:
    if dk_route not in _DK_ROUTES:
        raise ValueError("dk_route must be one of %s" % sorted(_DK_ROUTES))
    return ((IBWD_FLAG_DETERMINISTIC if deterministic else 0) | (IBWD_FLAG_ATOMIC_DK if atomic_dk else 0)
            | (IBWD_FLAG_BF16_OUT if bf16_out else 0) | _DK_ROUTES[dk_route])


def indexer_bwd_sparse(q, k, w, topk_ids, index_score, attn_score, d_q=None, d_w=None, d_k=None, *,
                       sm_scale: float = 1.0, grad_loss: float = 1.0, deterministic: bool = False,
                       atomic_dk: bool = False, global_ids: bool = False, bf16_out: bool = False,
                       dk_route: str = "auto", workspace=None, stream=None) -> Tuple:
    """Backward of the top-k indexer.  Returns (d_q, d_w, d_k), all fp32, or all
    bf16 with bf16_out (the fp32 results rounded to nearest even; not with atomic_dk).

    q [B,S_q,H,D] bf16, k [B,S_k,D] bf16, w [B,S_q,H] fp32, topk_ids [B,S_q,topk]
    int32, index_score / attn_score [B,S_q,topk] fp32.  Outputs are overwritten.
    atomic_dk selects the single-pass fp32-atomic dK route (no workspace).
    dk_route chooses between the deterministic routes: "auto" (by selection
    density), "key_ranges" or "slot_rows".
    global_ids: the ids index the flattened [B*S_k] keys; a row of batch b keeps
    only ids in [b*S_k, (b+1)*S_k), every other id is padding.
    """
    torch = _torch()
    B, S_q, H, D = q.shape
    S_k = k.shape[1]
    topk = topk_ids.shape[-1]
    _check(q, torch.bfloat16, (B, S_q, H, D), "q")
    _check(k, torch.bfloat16, (B, S_k, D), "k")
    _check(w, torch.float32, (B, S_q, H), "w")
    _check(topk_ids, torch.int32, (B, S_q, topk), "topk_ids")
    _check(index_score, torch.float32, (B, S_q, topk), "index_score")
    _check(attn_score, torch.float32, (B, S_q, topk), "attn_score")
    s = _stream(stream, q.device)
    d_q, d_w, d_k = _outputs(q, k, d_q, d_w, d_k, bf16_out, s)
    flags = _flags(deterministic, atomic_dk, bf16_out, dk_route) | (IBWD_FLAG_GLOBAL_IDS if global_ids else 0)
    workspace, ws_bytes = _workspace(False, B, S_q, S_k, H, D, topk, flags, workspace, q.device, s)
    st = library().indexer_bwd_sparse(
        _ptr(q), _ptr(k), _ptr(w), _ptr(topk_ids), _ptr(index_score), _ptr(attn_score), _ptr(d_q),
        _ptr(d_w), _ptr(d_k), B, S_q, S_k, H, D, topk, float(sm_scale), float(grad_loss), flags,
        _ptr(workspace), ws_bytes, int(s.cuda_stream))
    if st != IBWD_OK:
        raise IndexerBwdError(st)
    return d_q, d_w, d_k


def indexer_bwd_sparse_noalloc(q, k, w, topk_ids, index_score, attn_score, d_q, d_w, d_k, *,
                               sm_scale: float = 1.0, grad_loss: float = 1.0,
                               deterministic: bool = False, atomic_dk: bool = False,
                               global_ids: bool = False, bf16_out: bool = False,
                               dk_route: str = "auto", stream=None):
    """indexer_bwd_sparse through the allocation-free entry point: the library's
    own per-GPU scratch array (IBWD_NOALLOC_SCRATCH_BYTES) instead of a workspace.
    The outputs must be given (nothing is allocated here); returns them."""
    torch = _torch()
    if d_q is None or d_w is None or d_k is None:
        raise ValueError("indexer_bwd_sparse_noalloc allocates nothing: pass d_q, d_w and d_k")
    B, S_q, H, D = q.shape
    S_k = k.shape[1]
    topk = topk_ids.shape[-1]
    _check(q, torch.bfloat16, (B, S_q, H, D), "q")
    _check(k, torch.bfloat16, (B, S_k, D), "k")
    _check(w, torch.float32, (B, S_q, H), "w")
    _check(topk_ids, torch.int32, (B, S_q, topk), "topk_ids")
    _check(index_score, torch.float32, (B, S_q, topk), "index_score")
    _check(attn_score, torch.float32, (B, S_q, topk), "attn_score")
    dt = torch.bfloat16 if bf16_out else torch.float32
    for t, shp, name in zip((d_q, d_w, d_k), ((B, S_q, H, D), (B, S_q, H), (B, S_k, D)),
                            ("d_q", "d_w", "d_k")):
        _check(t, dt, shp, name)
    flags = _flags(deterministic, atomic_dk, bf16_out, dk_route) | (IBWD_FLAG_GLOBAL_IDS if global_ids else 0)
    s = _stream(stream, q.device)
    st = library().indexer_bwd_sparse_noalloc(
        _ptr(q), _ptr(k), _ptr(w), _ptr(topk_ids), _ptr(index_score), _ptr(attn_score), _ptr(d_q),
        _ptr(d_w), _ptr(d_k), B, S_q, S_k, H, D, topk, float(sm_scale), float(grad_loss), flags,
        int(s.cuda_stream))
    if st != IBWD_OK:
        raise IndexerBwdError(st)
    return d_q, d_w, d_k


def indexer_bwd_dense(q, k, w, index_score, attn_score, d_q=None, d_w=None, d_k=None, *,
                      q_offset: int = 0, sm_scale: float = 1.0, grad_loss: float = 1.0,
                      deterministic: bool = False, atomic_dk: bool = False,
                      bf16_out: bool = False, workspace=None, stream=None) -> Tuple:
    """Backward of the dense causal indexer (key s selected iff s <= t + q_offset).

    index_score / attn_score are [B,S_q,S_k] fp32.  Returns (d_q, d_w, d_k), fp32 or
    (bf16_out) bf16.
    """
    torch = _torch()
    B, S_q, H, D = q.shape
    S_k = k.shape[1]
    _check(q, torch.bfloat16, (B, S_q, H, D), "q")
    _check(k, torch.bfloat16, (B, S_k, D), "k")
    _check(w, torch.float32, (B, S_q, H), "w")
    _check(index_score, torch.float32, (B, S_q, S_k), "index_score")
    _check(attn_score, torch.float32, (B, S_q, S_k), "attn_score")
    s = _stream(stream, q.device)
    d_q, d_w, d_k = _outputs(q, k, d_q, d_w, d_k, bf16_out, s)
    flags = _flags(deterministic, atomic_dk, bf16_out)
    workspace, ws_bytes = _workspace(True, B, S_q, S_k, H, D, S_k, flags, workspace, q.device, s)
    st = library().indexer_bwd_dense(
        _ptr(q), _ptr(k), _ptr(w), _ptr(index_score), _ptr(attn_score), _ptr(d_q), _ptr(d_w),
        _ptr(d_k), B, S_q, S_k, H, D, int(q_offset), float(sm_scale), float(grad_loss), flags,
        _ptr(workspace), ws_bytes, int(s.cuda_stream))
    if st != IBWD_OK:
        raise IndexerBwdError(st)
    return d_q, d_w, d_k


def indexer_fwd_scores(q, k, w, scores=None, *, causal: bool = False, q_offset: int = 0,
                       stream=None):
    """Indexer scores [B,S_q,S_k] fp32: sum_h w*relu(q.k) for every key; with
    causal, keys s > t + q_offset score -inf.  q [B,S_q,H,D] bf16, k [B,S_k,D]
    bf16, w [B,S_q,H] fp32."""
    torch = _torch()
    B, S_q, H, D = q.shape
    S_k = k.shape[1]
    _check(q, torch.bfloat16, (B, S_q, H, D), "q")
    _check(k, torch.bfloat16, (B, S_k, D), "k")
    _check(w, torch.float32, (B, S_q, H), "w")
    s = _stream(stream, q.device)
    if scores is None:
        with torch.cuda.stream(s):
            scores = torch.empty((B, S_q, S_k), dtype=torch.float32, device=q.device)
    _check(scores, torch.float32, (B, S_q, S_k), "scores")
    st = library().indexer_fwd_scores(_ptr(q), _ptr(k), _ptr(w), _ptr(scores), B, S_q, S_k, H, D,
                                      int(bool(causal)), int(q_offset), int(s.cuda_stream))
    if st != IBWD_OK:
        raise IndexerBwdError(st)
    return scores


def indexer_topk(scores, topk: int, ids=None, values=None, *, stream=None):
    """Top-k of each row of scores [..., S_k] fp32: (ids int32, values fp32), each
    [..., topk]; ids ascending with -1 after the selected keys, values -inf there."""
    torch = _torch()
    S_k = scores.shape[-1]
    lead = tuple(scores.shape[:-1])
    rows = 1
    for n in lead:
        rows *= n
    _check(scores, torch.float32, lead + (S_k,), "scores")
    s = _stream(stream, scores.device)
    with torch.cuda.stream(s):
        if ids is None:
            ids = torch.empty(lead + (topk,), dtype=torch.int32, device=scores.device)
        if values is None:
            values = torch.empty(lead + (topk,), dtype=torch.float32, device=scores.device)
    _check(ids, torch.int32, lead + (topk,), "ids")
    _check(values, torch.float32, lead + (topk,), "values")
    st = library().indexer_topk(_ptr(scores), _ptr(ids), _ptr(values), rows, S_k, int(topk),
                                int(s.cuda_stream))
    if st != IBWD_OK:
        raise IndexerBwdError(st)
    return ids, values
