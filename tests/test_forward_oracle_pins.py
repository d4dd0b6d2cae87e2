"""Pins of the forward-score and top-k oracle (CPU) against facts outside its code:
brute-force loops on tiny inputs, the closed form where ReLU is the identity,
homogeneity, hand-worked selections (ties, masked keys, short rows) and the
order invariants of a top-k set.

Definition followed: the score I[t,s] = sum_h w[t,h]*relu(q[t,h,:].k[s,:]) whose
gradients the fp64 reference of the NVIDIA/cudnn-frontend PR #730 benchmark
harness computes; selection of the k largest finite scores per query row.
"""
import itertools

import numpy as np

import oracle


def brute_scores(q, k, w, q_offset=None):
    B, S_q, H, D = q.shape
    S_k = k.shape[1]
    out = np.zeros((B, S_q, S_k))
    for b, t, s in itertools.product(range(B), range(S_q), range(S_k)):
        if q_offset is not None and s > t + q_offset:
            out[b, t, s] = -np.inf
            continue
        tot = 0.0
        for h in range(H):
            dot = 0.0
            for d in range(D):
                dot += float(q[b, t, h, d]) * float(k[b, s, d])
            tot += float(w[b, t, h]) * max(dot, 0.0)
        out[b, t, s] = tot
    return out


def tiny(seed, B=2, S_q=5, S_k=7, H=3, D=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, S_q, H, D)), rng.standard_normal((B, S_k, D)),
            rng.standard_normal((B, S_q, H)))


def test_scores_brute_force():
    q, k, w = tiny(1)
    for off in (None, 0, 2, -1):
        got = oracle.forward_scores(q, k, w, off)
        ref = brute_scores(q, k, w, off)
        assert np.array_equal(np.isinf(got), np.isinf(ref))
        fin = np.isfinite(ref)
        assert np.allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12)
    assert np.isinf(oracle.forward_scores(q, k, w, -1)[:, 0, :]).all()   # row 0 sees no key


def test_scores_closed_form_all_positive():
    """q, k >= 0: ReLU is the identity and I = (sum_h w_h q_h) . k, one matmul."""
    rng = np.random.default_rng(2)
    q = np.abs(rng.standard_normal((1, 6, 5, 8)))
    k = np.abs(rng.standard_normal((1, 9, 8)))
    w = rng.standard_normal((1, 6, 5))
    wq = np.einsum("bth,bthd->btd", w, q)
    assert np.allclose(oracle.forward_scores(q, k, w), wq @ k.transpose(0, 2, 1), rtol=1e-12)


def test_scores_homogeneity():
    """relu is 1-homogeneous: I(a q) = a I(q) for a > 0, and I is linear in w."""
    q, k, w = tiny(3)
    base = oracle.forward_scores(q, k, w)
    assert np.allclose(oracle.forward_scores(2.5 * q, k, w), 2.5 * base, rtol=1e-12)
    assert np.allclose(oracle.forward_scores(q, k, -3.0 * w), -3.0 * base, rtol=1e-12)
    # a negative scale of q picks the other half-space of every dot product
    neg = oracle.forward_scores(-q, k, w)
    both = oracle.forward_scores(q, k, w) - neg
    wq = np.einsum("bth,bthd->bthd", w, q)
    lin = np.einsum("bthd,bsd->bts", wq, k)
    assert np.allclose(both, lin, rtol=1e-10, atol=1e-12)   # relu(x) - relu(-x) = x


def test_topk_hand_values():
    inf = np.inf
    rows = np.array([
        [0.5, 2.0, 2.0, -inf, 1.0, 2.0],      # three-way tie at the top: lower ids win
        [-inf, -inf, -inf, -inf, -inf, -inf],  # no candidate
        [-inf, 3.0, -inf, -1.0, -inf, -inf],  # fewer candidates than topk
        [-2.0, -1.0, -3.0, -0.5, -4.0, -1.0],  # negative scores, tie at the threshold
    ])
    ids, vals = oracle.select_topk(rows, 3)
    assert ids.tolist() == [[1, 2, 5], [-1, -1, -1], [1, 3, -1], [1, 3, 5]]
    assert vals[0].tolist() == [2.0, 2.0, 2.0]
    assert vals[2].tolist() == [3.0, -1.0, -inf]
    ids2, _ = oracle.select_topk(rows[:1], 2)
    assert ids2.tolist() == [[1, 2]]                       # the tie broken by key id
    ids6, _ = oracle.select_topk(rows[3:], 6)
    assert ids6.tolist() == [[0, 1, 2, 3, 4, 5]]          # topk = S_k keeps every key


def test_topk_invariants_random():
    rng = np.random.default_rng(4)
    sc = np.round(rng.standard_normal((40, 50)) * 4) / 4      # many ties
    sc[rng.random(sc.shape) < 0.2] = -np.inf
    for topk in (1, 7, 30, 50):
        ids, vals = oracle.select_topk(sc, topk)
        for r in range(sc.shape[0]):
            row = sc[r]
            cand = np.flatnonzero(np.isfinite(row))
            n = min(topk, cand.size)
            sel = ids[r, :n]
            assert (ids[r, n:] == -1).all() and np.isneginf(vals[r, n:]).all()
            assert (np.diff(sel) > 0).all()
            assert np.array_equal(vals[r, :n], row[sel])
            rest = np.setdiff1d(cand, sel)
            if rest.size and n:
                lo = row[sel].min()
                assert row[rest].max() <= lo
                # among keys scoring exactly the threshold, the selected ones have the lowest ids
                tied_rest = rest[row[rest] == lo]
                tied_sel = sel[row[sel] == lo]
                assert tied_rest.size == 0 or tied_sel.max() < tied_rest.min()
