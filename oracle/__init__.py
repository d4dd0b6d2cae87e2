"""fp64 CPU oracle of the lightning-indexer backward, and of the forward scores
and top-k selection that feed it (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never reaches it, and the two share no code.

The arithmetic lives in ``indexer_bwd_oracle.c`` (plain loops in fp64 that
follow the definition step by step); this module compiles it with gcc and
marshals numpy arrays.  bf16 inputs are widened to fp64 exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "indexer_bwd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        lp = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        dbl = ctypes.c_double
        lib.oracle_sparse.argtypes = [dp, dp, dp, ip, dp, dp] + [i64] * 6 + [dbl, dbl, dp, dp, dp]
        lib.oracle_sparse_rows.argtypes = [dp, dp, dp, ip, dp, dp] + [i64] * 6 + [dbl, dbl, i64, lp, dp, dp]
        lib.oracle_sparse_dk_rows.argtypes = [dp, dp, dp, ip, dp, dp] + [i64] * 6 + [dbl, dbl, i64, lp, dp]
        lib.oracle_dense.argtypes = [dp, dp, dp, dp, dp] + [i64] * 6 + [dbl, dbl, dp, dp, dp]
        lib.oracle_dense_rows.argtypes = [dp, dp, dp, dp, dp] + [i64] * 6 + [dbl, dbl, i64, lp, dp, dp]
        lib.oracle_dense_dk_rows.argtypes = [dp, dp, dp, dp, dp] + [i64] * 6 + [dbl, dbl, i64, lp, dp]
        lib.oracle_score_grad.argtypes = [ctypes.c_int, ip, dp, dp] + [i64] * 5 + [dbl, dbl, dp]
        for f in ("oracle_sparse", "oracle_sparse_rows", "oracle_sparse_dk_rows", "oracle_dense",
                  "oracle_dense_rows", "oracle_dense_dk_rows", "oracle_score_grad"):
            getattr(lib, f).restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _d(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def global_ids_to_local(ids, S_k: int) -> np.ndarray:
    """Batch-local ids of global top-k ids [B,S_q,topk].

    The benchmark harness of NVIDIA/cudnn-frontend PR #730 builds its kernel
    with topk_indices_global=True (at batch 1 only, where global and local ids
    coincide).  Read here: a global id indexes the keys of all batches laid end
    to end, so a row of batch b holds key id - b*S_k of its own batch when
    b*S_k <= id < (b+1)*S_k; any other id, a key of another batch included, is
    padding (-1), the same rule as for an out-of-range local id.
    """
    g = np.asarray(ids, dtype=np.int64)
    base = (np.arange(g.shape[0], dtype=np.int64) * S_k)[:, None, None]
    local = g - base
    return np.where((local >= 0) & (local < S_k), local, -1).astype(np.int32)


class Problem:
    """Inputs of one backward call, held as fp64 (ids int32, batch-local)."""

    def __init__(self, q, k, w, I, p, ids=None, *, S_k=None, sm_scale=1.0, grad_loss=1.0,
                 q_offset=0):
        self.q = _d(q)
        self.k = _d(k)
        self.w = _d(w)
        self.I = _d(I)
        self.p = _d(p)
        self.dense = ids is None
        self.ids = None if ids is None else np.ascontiguousarray(ids, dtype=np.int32)
        self.B, self.S_q, self.H, self.D = self.q.shape
        self.S_k = self.k.shape[1] if S_k is None else S_k
        self.topk = self.S_k if self.dense else self.ids.shape[-1]
        self.sm_scale = float(sm_scale)
        self.grad_loss = float(grad_loss)
        self.q_offset = int(q_offset)
        assert self.k.shape == (self.B, self.S_k, self.D)
        assert self.w.shape == (self.B, self.S_q, self.H)
        assert self.I.shape == (self.B, self.S_q, self.topk) == self.p.shape

    @classmethod
    def from_inputs(cls, x) -> "Problem":
        """From a ``synth.Inputs`` (bf16 bits for q/k, fp32 for w/I/p)."""
        return cls(widen_bf16(x.q), widen_bf16(x.k), x.w, x.index_score, x.attn_score, x.ids,
                   S_k=x.wl.S_k, sm_scale=x.sm_scale, grad_loss=x.grad_loss,
                   q_offset=x.wl.q_offset)

    def _head(self):
        dp = ctypes.c_double
        return (_ptr(self.q, dp), _ptr(self.k, dp), _ptr(self.w, dp))

    def _shape(self):
        return (self.B, self.S_q, self.S_k, self.H, self.D)

    def backward(self):
        """Full backward: (dq [B,S_q,H,D], dw [B,S_q,H], dk [B,S_k,D]) in fp64."""
        lib = _load()
        dq = np.zeros((self.B, self.S_q, self.H, self.D))
        dw = np.zeros((self.B, self.S_q, self.H))
        dk = np.zeros((self.B, self.S_k, self.D))
        dp = ctypes.c_double
        if self.dense:
            rc = lib.oracle_dense(*self._head(), _ptr(self.I, dp), _ptr(self.p, dp), *self._shape(),
                                  self.q_offset, self.sm_scale, self.grad_loss, _ptr(dq, dp),
                                  _ptr(dw, dp), _ptr(dk, dp))
        else:
            rc = lib.oracle_sparse(*self._head(), _ptr(self.ids, ctypes.c_int32), _ptr(self.I, dp),
                                   _ptr(self.p, dp), *self._shape(), self.topk, self.sm_scale,
                                   self.grad_loss, _ptr(dq, dp), _ptr(dw, dp), _ptr(dk, dp))
        if rc != 0:
            raise RuntimeError("oracle failed: %d" % rc)
        return dq, dw, dk

    def rows(self, rows: Sequence[int]):
        """dQ, dW of the listed rows (flat b*S_q + t): ([n,H,D], [n,H])."""
        lib = _load()
        r = np.ascontiguousarray(rows, dtype=np.int64)
        dq = np.zeros((len(r), self.H, self.D))
        dw = np.zeros((len(r), self.H))
        dp = ctypes.c_double
        lp = ctypes.c_int64
        if self.dense:
            rc = lib.oracle_dense_rows(*self._head(), _ptr(self.I, dp), _ptr(self.p, dp),
                                       *self._shape(), self.q_offset, self.sm_scale, self.grad_loss,
                                       len(r), _ptr(r, lp), _ptr(dq, dp), _ptr(dw, dp))
        else:
            rc = lib.oracle_sparse_rows(*self._head(), _ptr(self.ids, ctypes.c_int32),
                                        _ptr(self.I, dp), _ptr(self.p, dp), *self._shape(), self.topk,
                                        self.sm_scale, self.grad_loss, len(r), _ptr(r, lp),
                                        _ptr(dq, dp), _ptr(dw, dp))
        if rc != 0:
            raise RuntimeError("oracle failed: %d" % rc)
        return dq, dw

    def dk_rows(self, keys: Sequence[int]):
        """dK of the listed key rows (flat b*S_k + s): [n,D]."""
        lib = _load()
        kk = np.ascontiguousarray(keys, dtype=np.int64)
        dk = np.zeros((len(kk), self.D))
        dp = ctypes.c_double
        lp = ctypes.c_int64
        if self.dense:
            rc = lib.oracle_dense_dk_rows(*self._head(), _ptr(self.I, dp), _ptr(self.p, dp),
                                          *self._shape(), self.q_offset, self.sm_scale,
                                          self.grad_loss, len(kk), _ptr(kk, lp), _ptr(dk, dp))
        else:
            rc = lib.oracle_sparse_dk_rows(*self._head(), _ptr(self.ids, ctypes.c_int32),
                                           _ptr(self.I, dp), _ptr(self.p, dp), *self._shape(),
                                           self.topk, self.sm_scale, self.grad_loss, len(kk),
                                           _ptr(kk, lp), _ptr(dk, dp))
        if rc != 0:
            raise RuntimeError("oracle failed: %d" % rc)
        return dk

    def score_grad(self):
        """dI of every row: [B,S_q,topk] (dense: [B,S_q,S_k])."""
        lib = _load()
        dI = np.zeros(self.I.shape)
        dp = ctypes.c_double
        ids = self.ids if self.ids is not None else np.zeros(1, np.int32)
        rc = lib.oracle_score_grad(int(self.dense), _ptr(ids, ctypes.c_int32), _ptr(self.I, dp),
                                   _ptr(self.p, dp), self.B, self.S_q, self.S_k, self.topk,
                                   self.q_offset, self.sm_scale, self.grad_loss, _ptr(dI, dp))
        if rc != 0:
            raise RuntimeError("oracle failed: %d" % rc)
        return dI



# ---------------------------------------------------------------------------
# the step before the backward: indexer forward scores and top-k selection

def forward_scores(q, k, w, q_offset: Optional[int] = None, t_index=None) -> np.ndarray:
    """Indexer scores I [B,S_q,S_k] in fp64: I[t,s] = sum_h w[t,h]*relu(q[t,h,:].k[s,:]).

    This is the score whose gradients the fp64 `ref_grads` reference of the
    NVIDIA/cudnn-frontend PR #730 benchmark harness computes (its dW is the
    sum of g*relu(S), so dI/dw = relu(S)).  q_offset None: every key of the
    batch; otherwise key s is visible to query t iff s <= t + q_offset (the
    dense causal variant's rule) and masked keys score -inf.  t_index: the
    query index t of each row of q and w (default 0..S_q-1), for sampled rows.
    """
    q, k, w = _d(q), _d(k), _d(w)
    B, S_q, H, D = q.shape
    S_k = k.shape[1]
    out = np.empty((B, S_q, S_k))
    for b in range(B):
        S = np.matmul(q[b], k[b].T)                          # [S_q,H,S_k]
        out[b] = np.einsum("th,ths->ts", w[b], np.maximum(S, 0.0))
    if q_offset is not None:
        t = (np.arange(S_q) if t_index is None else np.asarray(t_index))[:, None]
        s = np.arange(S_k)[None, :]
        out[:, s > t + q_offset] = -np.inf
    return out


def select_topk(scores, topk: int):
    """Top-k selection of each row of scores [..., S_k]: (ids int32, values).

    Keys with a finite score are candidates; the row keeps its min(topk,
    candidates) largest, a tie going to the lower key id, listed in
    ascending key id; the remaining slots hold id -1 and value -inf.
    """
    sc = np.asarray(scores)
    lead = sc.shape[:-1]
    S_k = sc.shape[-1]
    flat = sc.reshape(-1, S_k)
    ids = np.full((flat.shape[0], topk), -1, dtype=np.int32)
    vals = np.full((flat.shape[0], topk), -np.inf, dtype=sc.dtype)
    key = np.arange(S_k)
    for r in range(flat.shape[0]):
        row = flat[r]
        cand = np.flatnonzero(np.isfinite(row))
        order = cand[np.lexsort((key[cand], -row[cand]))][:topk]   # score desc, then id asc
        keep = np.sort(order)
        ids[r, :keep.size] = keep
        vals[r, :keep.size] = row[keep]
    return ids.reshape(lead + (topk,)), vals.reshape(lead + (topk,))
