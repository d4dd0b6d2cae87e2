"""The allocation-free entry point (indexer_bwd_sparse_noalloc) against
indexer_bwd_sparse: two calls in a row on the library's scratch array, the
second smaller, each bitwise equal to the workspace call (same kernels, same
deterministic route, the key-range route at topk 1024 and the slot-row route
at topk 128 of 4096 keys); a call too large for the array is rejected before
anything is written."""
import dataclasses

import numpy as np
import pytest

from synth import WORKLOADS, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ibwd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_lightning_indexer_bwd_amd as m
    m.library()
    return m


def _dev(x):
    d = torch.device("cuda:0")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(d)

    return dict(q=bf16(x.q), k=bf16(x.k), w=torch.from_numpy(x.w).to(d),
                ids=torch.from_numpy(x.ids).to(d), I=torch.from_numpy(x.index_score).to(d),
                p=torch.from_numpy(x.attn_score).to(d))


def _outs(t, dt=torch.float32):
    B, S_q, H, D = t["q"].shape
    S_k = t["k"].shape[1]
    return (torch.full((B, S_q, H, D), float("nan"), dtype=dt, device="cuda:0"),
            torch.full((B, S_q, H), float("nan"), dtype=dt, device="cuda:0"),
            torch.full((B, S_k, D), float("nan"), dtype=dt, device="cuda:0"))


def _host(r):
    return [a.view(torch.int16).cpu().numpy() if a.dtype == torch.bfloat16 else a.cpu().numpy()
            for a in r]


@pytest.mark.parametrize("topk", [1024, 128])
@pytest.mark.parametrize("bf16_out", [False, True])
def test_noalloc_matches_workspace_call_twice(ibwd, bf16_out, topk):
    print(f"case: noalloc bf16_out={bf16_out} topk={topk}", flush=True)
    dt = torch.bfloat16 if bf16_out else torch.float32
    wl = dataclasses.replace(WORKLOADS["anchor"], topk=topk)
    assert ibwd.indexer_bwd_workspace_bytes(False, 1, 2048, 4096, 64, 128, topk, 0) <= \
        ibwd.IBWD_NOALLOC_SCRATCH_BYTES
    for S_q, seed, sm, gl in ((2048, 81, 1.0, 1.0), (300, 82, 0.7, 1.3)):
        x = make_inputs(wl, S_q=S_q, seed=seed)
        t = _dev(x)
        want = ibwd.indexer_bwd_sparse(t["q"], t["k"], t["w"], t["ids"], t["I"], t["p"],
                                       sm_scale=sm, grad_loss=gl, bf16_out=bf16_out)
        got = ibwd.indexer_bwd_sparse_noalloc(t["q"], t["k"], t["w"], t["ids"], t["I"], t["p"],
                                              *_outs(t, dt), sm_scale=sm, grad_loss=gl,
                                              bf16_out=bf16_out)
        torch.cuda.synchronize()
        for u, v in zip(_host(got), _host(want)):
            assert np.array_equal(u, v), S_q


def test_noalloc_rejects_calls_beyond_the_array(ibwd):
    print("case: noalloc too large", flush=True)
    x = make_inputs("anchor", S_q=2355, seed=83)   # one row past the array (H=64, D=128, topk=1024)
    t = _dev(x)
    assert ibwd.indexer_bwd_workspace_bytes(False, 1, 2355, 4096, 64, 128, 1024, 0) > \
        ibwd.IBWD_NOALLOC_SCRATCH_BYTES
    outs = _outs(t)
    with pytest.raises(ibwd.IndexerBwdError) as e:
        ibwd.indexer_bwd_sparse_noalloc(t["q"], t["k"], t["w"], t["ids"], t["I"], t["p"], *outs)
    assert e.value.status == ibwd.IBWD_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
    assert all(bool(torch.isnan(o).all()) for o in outs)   # untouched
