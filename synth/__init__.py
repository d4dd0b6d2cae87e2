"""Seeded synthetic inputs for the lightning-indexer backward.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It draws inputs only; it computes nothing of the backward pass
(no softmax gradient, no G, no dQ/dW/dK).  The one piece of indexer arithmetic
it holds is the forward index score used as the ``index_score`` input
(``I[t,j] = sum_h w[t,h] * relu(q[t,h,:] . k[id_j,:])``, evaluated in fp32 as
the workload description asks for "I recomputed fp32").

Workloads (NVIDIA/cudnn-frontend PR #730, the posted A/B harness: fixtures
with seeded randn q/k/w, per-row-unique ids, -1 padding; PR #549 anchor shape
B=1, H=64, D=128, S_k=4096, S_q=8192, topk=1024):

* ``tiny``    B=1 H=4  D=32  S_q=64   S_k=128  topk=16,   ~10% ids -1
* ``sparse``  B=1 H=64 D=128 S_q=4096 S_k=4096 topk=512,  no padding
* ``anchor``  B=1 H=64 D=128 S_q=8192 S_k=4096 topk=1024, 2% ids -1
* ``wide``    B=1 H=64 D=128 S_q=8192 S_k=4096 topk=2048, ids sorted per row
* ``dense``   B=1 H=64 D=128 S_q=S_k=4096, causal (every s <= t)

Generators: numpy ``Generator(PCG64(seed))`` with seed = 20260 + workload
index; q, k ~ N(0,1) rounded to bf16 (round-to-nearest-even); w ~ N(0,1)/sqrt(H)
in fp32; ids distinct per row (a uniform random permutation prefix); p is a
softmax of N(0,1) logits over the valid slots.  Padded slots carry garbage that
a correct backward must ignore: index_score 1e4, attn_score 0.123.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

PAD_INDEX_SCORE = 1.0e4
PAD_ATTN_SCORE = 0.123


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    H: int
    D: int
    S_q: int
    S_k: int
    topk: int           # dense: S_k (every key is a candidate, causal mask applies)
    pad_frac: float = 0.0
    sorted_ids: bool = False
    dense: bool = False
    q_offset: int = 0

    @property
    def seed(self) -> int:
        return 20260 + self.index

    def flops(self) -> float:
        """Algorithmic FLOP: three GEMMs of 2*H*D per selected (query, key) slot.

        Sparse counts the nominal topk per query (padding included); dense counts
        the t+1+q_offset keys of the causal row."""
        if self.dense:
            n = 0
            for t in range(self.S_q):
                n += max(0, min(t + self.q_offset, self.S_k - 1) + 1)
            return 6.0 * self.H * self.D * n * self.B
        return 6.0 * self.H * self.D * self.topk * self.S_q * self.B


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 4, 32, 64, 128, 16, pad_frac=0.10),
    "sparse": Workload("sparse", 1, 1, 64, 128, 4096, 4096, 512),
    "anchor": Workload("anchor", 2, 1, 64, 128, 8192, 4096, 1024, pad_frac=0.02),
    "wide": Workload("wide", 3, 1, 64, 128, 8192, 4096, 2048, sorted_ids=True),
    "dense": Workload("dense", 4, 1, 64, 128, 4096, 4096, 4096, dense=True),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    wl: Workload
    q: np.ndarray        # uint16 bf16 bits [B,S_q,H,D]
    k: np.ndarray        # uint16 bf16 bits [B,S_k,D]
    w: np.ndarray        # fp32 [B,S_q,H]
    ids: Optional[np.ndarray]   # int32 [B,S_q,topk] (None for dense)
    index_score: np.ndarray     # fp32 [B,S_q,topk] or [B,S_q,S_k]
    attn_score: np.ndarray      # fp32 same shape
    sm_scale: float = 1.0
    grad_loss: float = 1.0


def _draw_ids(rng: np.random.Generator, S_q: int, S_k: int, topk: int) -> np.ndarray:
    # per-row distinct ids: the first topk entries of an argsort of uniforms
    # (a uniform random permutation prefix); rows in blocks to bound memory
    out = np.empty((S_q, topk), dtype=np.int32)
    blk = 512
    for r0 in range(0, S_q, blk):
        r1 = min(S_q, r0 + blk)
        u = rng.random((r1 - r0, S_k), dtype=np.float32)
        out[r0:r1] = np.argpartition(u, topk - 1, axis=1)[:, :topk] if topk < S_k else np.argsort(u, axis=1)
    return out


def _softmax_rows(logits: np.ndarray, valid: np.ndarray) -> np.ndarray:
    z = np.where(valid, logits, -np.inf)
    m = z.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(valid, np.exp(z - m), 0.0)
    s = e.sum(axis=-1, keepdims=True)
    s = np.where(s > 0, s, 1.0)
    return e / s


def forward_index_score_sparse(q_bits, k_bits, w, ids, S_k, device="cpu", block=256):
    """I[b,t,j] = sum_h w[b,t,h] * relu(q[b,t,h,:] . k[b,id,:]) in fp32 (valid slots only)."""
    import torch
    B, S_q, H, D = q_bits.shape
    topk = ids.shape[-1]
    out = np.zeros((B, S_q, topk), dtype=np.float32)
    for b in range(B):
        kf = torch.from_numpy(bf16_to_f32(k_bits[b])).to(device)
        for t0 in range(0, S_q, block):
            t1 = min(S_q, t0 + block)
            qf = torch.from_numpy(bf16_to_f32(q_bits[b, t0:t1])).to(device)          # [n,H,D]
            idb = torch.from_numpy(ids[b, t0:t1].astype(np.int64)).to(device)        # [n,topk]
            valid = (idb >= 0) & (idb < S_k)
            kg = kf[idb.clamp(0, S_k - 1)]                                           # [n,topk,D]
            s = torch.bmm(qf, kg.transpose(1, 2).contiguous())                       # [n,H,topk]
            wf = torch.from_numpy(w[b, t0:t1]).to(device)
            i = (torch.relu(s) * wf[:, :, None]).sum(dim=1)
            i = torch.where(valid, i, torch.zeros_like(i))
            out[b, t0:t1] = i.cpu().numpy()
    return out


def forward_index_score_dense(q_bits, k_bits, w, device="cpu", block=128):
    """I[b,t,s] for every (t,s) in fp32 (the causal mask is applied by the caller)."""
    import torch
    B, S_q, H, D = q_bits.shape
    S_k = k_bits.shape[1]
    out = np.zeros((B, S_q, S_k), dtype=np.float32)
    for b in range(B):
        kf = torch.from_numpy(bf16_to_f32(k_bits[b])).to(device)
        for t0 in range(0, S_q, block):
            t1 = min(S_q, t0 + block)
            qf = torch.from_numpy(bf16_to_f32(q_bits[b, t0:t1])).to(device).reshape(-1, D)
            s = (qf @ kf.t().contiguous()).reshape(t1 - t0, H, S_k)
            wf = torch.from_numpy(w[b, t0:t1]).to(device)
            out[b, t0:t1] = (torch.relu(s) * wf[:, :, None]).sum(dim=1).cpu().numpy()
    return out


def make_inputs(wl: Workload | str, *, seed: Optional[int] = None, device="cpu",
                grad_loss: float = 1.0, sm_scale: float = 1.0, pad_frac: Optional[float] = None,
                S_q: Optional[int] = None) -> Inputs:
    """Draw one workload.  ``S_q`` may shrink the query count (same generators)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if S_q is not None:
        wl = dataclasses.replace(wl, S_q=S_q)
    if pad_frac is not None:
        wl = dataclasses.replace(wl, pad_frac=pad_frac)
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    B, H, D, S_q, S_k = wl.B, wl.H, wl.D, wl.S_q, wl.S_k
    q = bf16_round(rng.standard_normal((B, S_q, H, D), dtype=np.float32))
    k = bf16_round(rng.standard_normal((B, S_k, D), dtype=np.float32))
    w = (rng.standard_normal((B, S_q, H), dtype=np.float32) / np.float32(math.sqrt(H))).astype(np.float32)
    if wl.dense:
        t = np.arange(S_q)[:, None]
        s = np.arange(S_k)[None, :]
        valid = np.broadcast_to(s <= t + wl.q_offset, (B, S_q, S_k))
        I = forward_index_score_dense(q, k, w, device=device)
        logits = rng.standard_normal((B, S_q, S_k), dtype=np.float32).astype(np.float64)
        p = _softmax_rows(logits, valid).astype(np.float32)
        I = np.where(valid, I, np.float32(PAD_INDEX_SCORE)).astype(np.float32)
        p = np.where(valid, p, np.float32(PAD_ATTN_SCORE)).astype(np.float32)
        return Inputs(wl, q, k, w, None, I, p, sm_scale, grad_loss)
    ids = np.stack([_draw_ids(rng, S_q, S_k, wl.topk) for _ in range(B)])
    if wl.sorted_ids:
        ids = np.sort(ids, axis=-1)
    if wl.pad_frac > 0:
        pad = rng.random(ids.shape) < wl.pad_frac
        ids = np.where(pad, np.int32(-1), ids).astype(np.int32)
    valid = (ids >= 0) & (ids < S_k)
    I = forward_index_score_sparse(q, k, w, ids, S_k, device=device)
    logits = rng.standard_normal(ids.shape, dtype=np.float32).astype(np.float64)
    p = _softmax_rows(logits, valid).astype(np.float32)
    I = np.where(valid, I, np.float32(PAD_INDEX_SCORE)).astype(np.float32)
    p = np.where(valid, p, np.float32(PAD_ATTN_SCORE)).astype(np.float32)
    return Inputs(wl, q, k, w, ids.astype(np.int32), I, p, sm_scale, grad_loss)
