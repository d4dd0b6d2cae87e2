"""GPU parity of the indexer forward scores and the top-k selection (through the
C ABI) against the fp64 oracle.

Scores: bf16 products are exact in fp32, the MFMA accumulates D of them and the
epilogue sums H weighted terms, so each score is within
(D + H + 8) * 2^-24 * sum_h |w_h| * sum_d |q_hd k_d| of the exact value (the
bound used below, doubled); masked keys are -inf on both sides.
Top-k: an integer decision taken on the kernel's own fp32 scores, so it is
compared bit for bit with the oracle's selection of the same fp32 values.
"""
import numpy as np
import pytest

import oracle
from synth import make_inputs, WORKLOADS
from tests.util import relrms

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ibwd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_lightning_indexer_bwd_amd as m
    m.library()
    return m


def log(msg):
    print(msg, flush=True)


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def draw(seed, B, S_q, S_k, H, D):
    """q, k as bf16 bit patterns and fp64 values, w fp32 (the synth recipe: N(0,1), w / 8)."""
    rng = np.random.default_rng(seed)
    qf = rng.standard_normal((B, S_q, H, D)).astype(np.float32)
    kf = rng.standard_normal((B, S_k, D)).astype(np.float32)
    w = (rng.standard_normal((B, S_q, H)) / 8).astype(np.float32)
    qb = torch.from_numpy(qf).to(torch.bfloat16)
    kb = torch.from_numpy(kf).to(torch.bfloat16)
    return (qb.view(torch.int16).numpy().view(np.uint16), kb.view(torch.int16).numpy().view(np.uint16),
            qb.double().numpy(), kb.double().numpy(), w)


def check_scores(got, q64, k64, w, q_offset, t_index=None):
    ref = oracle.forward_scores(q64, k64, w, q_offset, t_index)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    assert np.isfinite(got[fin]).all()
    H, D = q64.shape[2], q64.shape[3]
    mag = np.einsum("bth,bths->bts", np.abs(w).astype(np.float64),
                    np.abs(q64) @ np.abs(k64).transpose(0, 2, 1)[:, None])
    tol = 2 * (D + H + 8) * 2.0 ** -24 * mag
    err = np.abs(got.astype(np.float64) - np.where(fin, ref, 0.0))
    assert (err[fin] <= tol[fin]).all(), float((err[fin] / tol[fin]).max())
    log(f"  scores relRMS {relrms(got[fin], ref[fin]):.3e}, max err/bound "
        f"{float((err[fin] / np.maximum(tol[fin], 1e-300)).max()):.3f}")
    return ref


@pytest.mark.parametrize("B,S_q,S_k,H,D,causal,q_offset", [
    (1, 40, 300, 64, 128, False, 0),     # ragged queries (5 workgroups) and keys (not a tile multiple)
    (2, 21, 200, 33, 64, True, 0),       # two head tiles, the second mostly padding; causal
    (1, 17, 130, 8, 32, True, -5),       # negative offset: the first rows see no key
    (1, 64, 512, 64, 128, True, 100),
    (3, 9, 65, 1, 32, False, 0),         # one head; one key past a tile
    (1, 24, 700, 40, 32, True, 3),       # D=32 with two head tiles; keys past a 256-key tile
    (2, 16, 1000, 20, 128, False, 0),    # D=128 with one head tile
])
def test_fwd_scores_small(ibwd, B, S_q, S_k, H, D, causal, q_offset):
    log(f"case: fwd scores B={B} S_q={S_q} S_k={S_k} H={H} D={D} causal={causal} off={q_offset}")
    qb, kb, q64, k64, w = draw(S_q * 7 + S_k, B, S_q, S_k, H, D)
    sc = ibwd.indexer_fwd_scores(bf16_dev(qb), bf16_dev(kb), torch.from_numpy(w).cuda(),
                                 causal=causal, q_offset=q_offset)
    torch.cuda.synchronize()
    check_scores(sc.cpu().numpy(), q64, k64, w, q_offset if causal else None)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_scores_full_size_sampled_rows(ibwd, causal):
    """S_q=8192, S_k=4096, H=64, D=128 (the anchor shapes): 48 sampled query rows
    against the oracle, every key of each."""
    log(f"case: fwd scores full size causal={causal}")
    wl = WORKLOADS["anchor"]
    qb, kb, q64, k64, w = draw(5, 1, wl.S_q, wl.S_k, wl.H, wl.D)
    sc = ibwd.indexer_fwd_scores(bf16_dev(qb), bf16_dev(kb), torch.from_numpy(w).cuda(),
                                 causal=causal, q_offset=0)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, 1, 63, 64, wl.S_q - 1, np.random.default_rng(1).integers(0, wl.S_q, 43)])
    got = sc[:, torch.from_numpy(rows).cuda()].cpu().numpy()
    check_scores(got, q64[:, rows], k64, w[:, rows], 0 if causal else None, t_index=rows)


def topk_dev(ibwd, scores, topk):
    ids, vals = ibwd.indexer_topk(scores, topk)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), vals.cpu().numpy()


def check_topk(ibwd, scores, topk):
    ids, vals = topk_dev(ibwd, scores, topk)
    rid, rval = oracle.select_topk(scores.cpu().numpy().astype(np.float64), topk)
    assert np.array_equal(ids, rid)
    assert np.array_equal(vals.astype(np.float64), rval)
    return ids


@pytest.mark.parametrize("topk", [1, 37, 256, 300])
def test_topk_of_forward_scores(ibwd, topk):
    """Top-k of the kernel's own causal scores: rows with fewer visible keys than
    topk pad with -1."""
    log(f"case: topk of scores topk={topk}")
    qb, kb, _, _, w = draw(11, 2, 50, 300, 16, 64)
    sc = ibwd.indexer_fwd_scores(bf16_dev(qb), bf16_dev(kb), torch.from_numpy(w).cuda(),
                                 causal=True, q_offset=20)
    ids = check_topk(ibwd, sc, topk)
    assert (ids[:, 0, min(topk, 21):] == -1).all()


@pytest.mark.parametrize("S_k", [1000, 2000, 4096, 5000])
def test_topk_ties_signed_zero_and_non_finite(ibwd, S_k):
    """Heavy ties (values on a coarse grid), +0 and -0, -inf, +inf and NaN (not
    candidates), all-masked rows, a row of equal values; rows held in registers
    (S_k <= 4096, three sizes) and rows read from memory per pass (5000)."""
    log(f"case: topk ties and special values S_k={S_k}")
    rng = np.random.default_rng(7)
    rows = 24
    x = (np.round(rng.standard_normal((rows, S_k)) * 2) / 2).astype(np.float32)
    x[rng.random(x.shape) < 0.1] = -np.inf
    x[rng.random(x.shape) < 0.02] = np.inf
    x[rng.random(x.shape) < 0.02] = np.nan
    x[rng.random(x.shape) < 0.05] = -0.0
    x[3] = -np.inf
    x[4, :] = 0.0
    x[4, ::3] = -0.0
    x[5, 7:] = np.nan
    x[6, :] = 1.5                     # every key equal
    x[7, :] = np.float32(3.0e38)      # equal and near the largest float
    x[7, ::5] = -np.float32(3.0e38)
    sc = torch.from_numpy(x).cuda()
    for topk in (1, 64, S_k // 2, S_k - 1, S_k):
        check_topk(ibwd, sc, topk)


def test_topk_long_rows(ibwd):
    log("case: topk long rows")
    rng = np.random.default_rng(8)
    x = rng.standard_normal((6, 70001)).astype(np.float32)
    sc = torch.from_numpy(x).cuda()
    for topk in (2048, 70001):
        check_topk(ibwd, sc, topk)


def test_topk_full_size_and_into_backward(ibwd):
    """Top-k 1024 of 8192 x 4096 forward scores (the anchor shapes), every row
    against the oracle; then the selected ids and scores are the backward's
    topk_ids and index_score, checked on sampled rows against the oracle's
    backward of the same selection."""
    log("case: topk full size + backward")
    wl = WORKLOADS["anchor"]
    x = make_inputs("anchor", seed=3, device="cuda:0")
    q, k = bf16_dev(x.q), bf16_dev(x.k)
    w = torch.from_numpy(x.w).cuda()
    sc = ibwd.indexer_fwd_scores(q, k, w)
    ids = check_topk(ibwd, sc, wl.topk)
    assert (ids >= 0).all()
    ids_d, vals_d = ibwd.indexer_topk(sc, wl.topk)
    p = torch.softmax(torch.randn(vals_d.shape, device="cuda:0", generator=torch.Generator(
        device="cuda:0").manual_seed(4)), dim=-1)
    dq, dw, _ = ibwd.indexer_bwd_sparse(q, k, w, ids_d, vals_d, p)
    torch.cuda.synchronize()
    prob = oracle.Problem(oracle.widen_bf16(x.q), oracle.widen_bf16(x.k), x.w, vals_d.cpu().numpy(),
                          p.cpu().numpy(), ids_d.cpu().numpy(), S_k=wl.S_k)
    rows = np.sort(np.random.default_rng(2).choice(wl.S_q, size=24, replace=False))
    rq, rw = prob.rows(rows)
    dq = dq.cpu().numpy()[0, rows]
    dw = dw.cpu().numpy()[0, rows]
    log(f"  backward of the selection: dq relRMS {relrms(dq, rq):.3e}, dw {relrms(dw, rw):.3e}")
    assert relrms(dq, rq) <= 2e-3 and relrms(dw, rw) <= 2e-3
