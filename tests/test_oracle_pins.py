"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test fixes part of the oracle to something independent of its code:
finite differences of the KL loss (every gradient, the softmax gradient and
the padding rules together), closed forms where ReLU is the identity (textbook
matmul / index_add), the Euler identities of a 1-homogeneous score, the
zero-sum of a softmax gradient, a two-slot sigmoid closed form, a hand-worked
example, padding equivalence and the dense-vs-sparse cross entry.

Definition followed (NVIDIA/cudnn-frontend PR #730, posted benchmark harness:
the fp64 `ref_grads` reference and the padding battery; PR #549: dK is an fp32
scatter-add, dQ/dW deterministic).
"""
import json
import os

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
from synth import make_inputs
from tests.util import relrms

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# an independent forward + loss, written here in numpy (fp64)

def fwd_scores(q, k, w, key_of):
    """S [B,S_q,H,n] and I [B,S_q,n] for slots key_of [B,S_q,n] (-1 = padding)."""
    B, S_q, H, D = q.shape
    kg = np.take_along_axis(k[:, None, :, :], np.clip(key_of, 0, None)[..., None], axis=2)
    S = np.einsum("bthd,btnd->bthn", q, kg)
    I = np.einsum("bth,bthn->btn", w, np.maximum(S, 0.0))
    return S, np.where(key_of >= 0, I, 0.0)


def kl_loss(q, k, w, key_of, p, sm_scale, grad_loss):
    """grad_loss * sum_rows KL(p || softmax_V(sm_scale * I(q,k,w)))."""
    _, I = fwd_scores(q, k, w, key_of)
    valid = key_of >= 0
    total = 0.0
    for b in range(q.shape[0]):
        for t in range(q.shape[1]):
            v = valid[b, t]
            if not v.any():
                continue
            z = sm_scale * I[b, t, v]
            logP = z - (z.max() + np.log(np.exp(z - z.max()).sum()))
            pv = p[b, t, v]
            total += float(np.sum(pv * (np.log(pv) - logP)))
    return grad_loss * total


def sparse_key_of(ids, S_k):
    return np.where((ids >= 0) & (ids < S_k), ids, -1)


def dense_key_of(B, S_q, S_k, q_offset):
    s = np.arange(S_k)[None, :]
    t = np.arange(S_q)[:, None]
    return np.broadcast_to(np.where(s <= t + q_offset, s, -1), (B, S_q, S_k)).copy()


def random_p(rng, key_of, garbage=0.123):
    valid = key_of >= 0
    x = np.where(valid, rng.random(key_of.shape) + 0.05, 0.0)
    s = x.sum(-1, keepdims=True)
    x = x / np.where(s > 0, s, 1.0)
    return np.where(valid, x, garbage)


def draw_kinkfree(rng, B, S_q, S_k, H, D, key_of, margin=1e-3):
    for _ in range(200):
        q = rng.standard_normal((B, S_q, H, D))
        k = rng.standard_normal((B, S_k, D))
        S, _ = fwd_scores(q, k, np.ones((B, S_q, H)), key_of)
        if np.abs(S[np.broadcast_to((key_of >= 0)[:, :, None, :], S.shape)]).min() > margin:
            return q, k
    raise RuntimeError("could not draw kink-free inputs")


def fd_grad(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


def check_fd(q, k, w, key_of, p, sm_scale, grad_loss, grads):
    def loss():
        return kl_loss(q, k, w, key_of, p, sm_scale, grad_loss)
    dq, dw, dk = grads
    for name, x, g in (("dq", q, dq), ("dw", w, dw), ("dk", k, dk)):
        num = fd_grad(loss, x)
        scale = max(np.abs(num).max(), 1e-3)
        err = np.abs(num - g).max() / scale
        assert err < 1e-6, f"{name}: finite-difference mismatch {err:.3e}"


# ---------------------------------------------------------------------------

@pytest.mark.parametrize("sm_scale,grad_loss", [(1.0, 1.0), (0.7, 1.5), (1.3, 0.5)])
def test_fd_sparse(sm_scale, grad_loss):
    """Finite differences of the KL loss pin dQ, dW, dK, the softmax gradient,
    the padding rules (-1, negative, positive out-of-range, batch-local ids) and
    duplicate ids (independent slots)."""
    rng = np.random.default_rng(7)
    B, S_q, S_k, H, D, topk = 2, 3, 6, 3, 4, 6
    ids = np.array([[[0, 5, -1, 2, 2, 7],      # duplicate 2, OOB 7 (= key 1 of batch 1 if flattened)
                     [1, 3, 4, -1, -5, 0],
                     [-1, -1, -1, -1, -1, -1]],  # all padding
                    [[5, 4, 3, 2, 1, 0],
                     [0, 6, 1, -1, 5, 5],
                     [2, 3, 12, 4, -1, 1]]], dtype=np.int32)
    key_of = sparse_key_of(ids, S_k)
    q, k = draw_kinkfree(rng, B, S_q, S_k, H, D, key_of)
    w = rng.standard_normal((B, S_q, H))
    _, I = fwd_scores(q, k, w, key_of)
    I = np.where(key_of >= 0, I, 1e4)
    p = random_p(rng, key_of)
    prob = oracle.Problem(q, k, w, I, p, ids, S_k=S_k, sm_scale=sm_scale, grad_loss=grad_loss)
    grads = prob.backward()
    check_fd(q, k, w, key_of, p, sm_scale, grad_loss, grads)
    # the all-padding row contributes nothing
    assert np.all(grads[0][0, 2] == 0) and np.all(grads[1][0, 2] == 0)


@pytest.mark.parametrize("q_offset", [0, 1, -2, 9])
def test_fd_dense(q_offset):
    """Finite differences pin the dense causal variant, including the inclusive
    s <= t + q_offset boundary and rows whose key set is empty."""
    rng = np.random.default_rng(11 + q_offset)
    B, S_q, S_k, H, D = 1, 5, 6, 3, 4
    key_of = dense_key_of(B, S_q, S_k, q_offset)
    q, k = draw_kinkfree(rng, B, S_q, S_k, H, D, key_of)
    w = rng.standard_normal((B, S_q, H))
    _, I = fwd_scores(q, k, w, key_of)
    I = np.where(key_of >= 0, I, 1e4)
    p = random_p(rng, key_of)
    prob = oracle.Problem(q, k, w, I, p, None, q_offset=q_offset, sm_scale=0.9, grad_loss=1.2)
    check_fd(q, k, w, key_of, p, 0.9, 1.2, prob.backward())


def test_closed_form_all_positive():
    """With q, k > 0 every score is positive, ReLU is the identity and the
    backward reduces to plain products: dQ = w * (dI @ K_g), dW = q . (dI @ K_g),
    dK = index_add(dI_j * sum_h w_h q_h); dI from scipy's softmax."""
    rng = np.random.default_rng(3)
    B, S_q, S_k, H, D, topk = 1, 4, 9, 5, 6, 7
    q = rng.random((B, S_q, H, D)) + 0.1
    k = rng.random((B, S_k, D)) + 0.1
    w = rng.standard_normal((B, S_q, H))
    ids = np.stack([np.stack([rng.permutation(S_k)[:topk] for _ in range(S_q)])]).astype(np.int32)
    I = rng.standard_normal((B, S_q, topk)) * 3
    p = softmax(rng.standard_normal((B, S_q, topk)), axis=-1)
    dq, dw, dk = oracle.Problem(q, k, w, I, p, ids, S_k=S_k, grad_loss=1.7).backward()
    dI = 1.7 * (softmax(I, axis=-1) - p)
    dq_ref = np.zeros_like(dq)
    dw_ref = np.zeros_like(dw)
    dk_ref = np.zeros_like(dk)
    for t in range(S_q):
        kg = k[0, ids[0, t]]                      # [topk, D]
        v = dI[0, t] @ kg                         # [D]
        dq_ref[0, t] = w[0, t][:, None] * v[None, :]
        dw_ref[0, t] = q[0, t] @ v
        np.add.at(dk_ref[0], ids[0, t], np.outer(dI[0, t], w[0, t] @ q[0, t]))
    np.testing.assert_allclose(dq, dq_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dw, dw_ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk, dk_ref, rtol=1e-12, atol=1e-13)


def test_euler_identities_tiny_workload():
    """ReLU is 1-homogeneous: <q[t,h], dQ[t,h]> = w[t,h] dW[t,h] for every (t,h),
    and sum_s <k_s, dK_s> = sum_{t,h} w dW = sum_{t,j} dI_j I_j when I is the
    forward of the same q, k, w."""
    x = make_inputs("tiny")
    prob = oracle.Problem.from_inputs(x)
    key_of = sparse_key_of(x.ids, x.wl.S_k)
    _, I64 = fwd_scores(prob.q, prob.k, prob.w, key_of)
    prob.I = np.ascontiguousarray(np.where(key_of >= 0, I64, 1e4))
    dq, dw, dk = prob.backward()
    lhs = np.einsum("bthd,bthd->bth", prob.q, dq)
    np.testing.assert_allclose(lhs, prob.w * dw, rtol=1e-10, atol=1e-13)
    tot_k = float(np.sum(prob.k * dk))
    tot_w = float(np.sum(prob.w * dw))
    dI = prob.score_grad()
    tot_i = float(np.sum(np.where(key_of >= 0, dI * I64, 0.0)))
    assert abs(tot_k - tot_w) <= 1e-11 * max(1.0, abs(tot_w))
    assert abs(tot_i - tot_w) <= 1e-11 * max(1.0, abs(tot_w))


def test_score_grad_invariants():
    """dI sums to zero over the valid slots (up to 1 - sum p), is zero on padding, equals
    grad_loss*sm_scale*(softmax - p) (scipy) and is linear in grad_loss."""
    x = make_inputs("tiny")
    prob = oracle.Problem.from_inputs(x)
    prob.sm_scale = 0.8
    prob.grad_loss = 1.5
    dI = prob.score_grad()
    valid = (x.ids >= 0) & (x.ids < x.wl.S_k)
    assert np.all(dI[~valid] == 0)
    # sum_V dI = grad_loss*sm_scale*(1 - sum_V p): zero when p is normalised over V
    # (the fp32 attn_score of the workload sums to 1 only up to fp32 rounding)
    psum = np.where(valid, prob.p, 0).sum(-1)
    assert np.abs(np.where(valid, dI, 0).sum(-1) - 1.5 * 0.8 * (1.0 - psum)).max() < 1e-15
    z = np.where(valid, 0.8 * prob.I, -np.inf)
    ref = 1.5 * 0.8 * (softmax(z, axis=-1) - np.where(valid, prob.p, 0))
    np.testing.assert_allclose(dI, np.where(valid, ref, 0), rtol=1e-12, atol=1e-15)


def test_two_slot_sigmoid():
    """topk = 2: dI_1 = grad_loss * sm_scale * (sigmoid(z_1 - z_2) - p_1), dI_2 = -dI_1."""
    I = np.array([[[0.3, -1.1]]])
    p = np.array([[[0.25, 0.75]]])
    ids = np.array([[[0, 1]]], dtype=np.int32)
    q = np.ones((1, 1, 1, 1))
    k = np.ones((1, 2, 1))
    prob = oracle.Problem(q, k, np.ones((1, 1, 1)), I, p, ids, S_k=2, sm_scale=1.7, grad_loss=0.6)
    dI = prob.score_grad()[0, 0]
    e = 0.6 * 1.7 * (expit(1.7 * (0.3 + 1.1)) - 0.25)
    assert abs(dI[0] - e) < 1e-15 and abs(dI[1] + e) < 1e-15


def test_uniform_special_case_is_zero():
    """I constant over V and p uniform over V: softmax(I) = p, so every gradient is 0."""
    rng = np.random.default_rng(5)
    B, S_q, S_k, H, D, topk = 1, 3, 8, 2, 3, 5
    ids = np.array([[[0, 1, 2, -1, 3], [4, 5, 6, 7, 0], [-1, 2, 2, 9, 1]]], dtype=np.int32)
    key_of = sparse_key_of(ids, S_k)
    nvalid = (key_of >= 0).sum(-1, keepdims=True)
    p = np.where(key_of >= 0, 1.0 / nvalid, 0.5)
    I = np.where(key_of >= 0, 2.5, -7.0)
    q = rng.standard_normal((B, S_q, H, D))
    k = rng.standard_normal((B, S_k, D))
    w = rng.standard_normal((B, S_q, H))
    dq, dw, dk = oracle.Problem(q, k, w, I, p, ids, S_k=S_k).backward()
    assert np.abs(dq).max() < 1e-15 and np.abs(dw).max() < 1e-15 and np.abs(dk).max() < 1e-15


def test_linear_in_grad_loss():
    x = make_inputs("tiny")
    prob = oracle.Problem.from_inputs(x)
    a = prob.backward()
    prob.grad_loss = 1.5
    b = prob.backward()
    for u, v in zip(a, b):
        np.testing.assert_allclose(v, 1.5 * u, rtol=1e-13, atol=1e-16)


def test_hand_worked_example():
    """A one-query example worked by hand from the definition (tests/golden)."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    prob = oracle.Problem(np.array(g["q"]), np.array(g["k"]), np.array(g["w"]), np.array(g["I"]),
                          np.array(g["p"]), np.array(g["ids"], dtype=np.int32), S_k=g["S_k"],
                          sm_scale=g["sm_scale"], grad_loss=g["grad_loss"])
    dq, dw, dk = prob.backward()
    np.testing.assert_allclose(prob.score_grad(), np.array(g["dI"]), atol=1e-15)
    np.testing.assert_allclose(dq, np.array(g["dq"]), atol=1e-14)
    np.testing.assert_allclose(dw, np.array(g["dw"]), atol=1e-14)
    np.testing.assert_allclose(dk, np.array(g["dk"]), atol=1e-14)


def test_padding_equivalence():
    """-1, other negatives and positive out-of-range ids are all padding, and
    whatever I/p hold there is ignored: the outputs are bitwise equal
    (analogue of the PR #730 padding-equivalence battery)."""
    x = make_inputs("tiny")
    base = oracle.Problem.from_inputs(x)
    ref = base.backward()
    pad = x.ids == -1
    assert pad.any()
    ids2 = x.ids.copy()
    n = np.arange(ids2.size).reshape(ids2.shape)
    ids2[pad] = np.where(n[pad] % 3 == 0, x.wl.S_k + (n[pad] % 9999), np.where(n[pad] % 3 == 1, -7, -1))
    I2 = base.I.copy()
    p2 = base.p.copy()
    I2[pad] = -3e3
    p2[pad] = 0.777
    alt = oracle.Problem(base.q, base.k, base.w, I2, p2, ids2, S_k=x.wl.S_k).backward()
    for u, v in zip(ref, alt):
        assert np.array_equal(u, v)


def test_global_ids_remap_hand_values():
    """Global ids (topk_indices_global of the PR #730 harness) read as indices
    into the keys of all batches laid end to end: hand-computed local ids for
    B=2, S_k=3, with another batch's keys, -1, and the int32 extremes."""
    row = [0, 2, 3, -1, 5, 6, 2**31 - 1, -2**31]
    ids = np.array([[row], [row]], dtype=np.int32)
    got = oracle.global_ids_to_local(ids, 3)
    assert got.dtype == np.int32
    assert got[0, 0].tolist() == [0, 2, -1, -1, -1, -1, -1, -1]
    assert got[1, 0].tolist() == [-1, -1, 0, -1, 2, -1, -1, -1]
    # at one batch, global and local ids coincide (out-of-range ids stay padding)
    one = oracle.global_ids_to_local(ids[:1], 3)
    assert one[0, 0].tolist() == [0, 2, -1, -1, -1, -1, -1, -1]


def test_dense_equals_sparse_cross_entry():
    """dense(q,k,w,I,p) equals sparse with ids[t,j] = j if j <= t + q_offset else -1."""
    rng = np.random.default_rng(9)
    B, S_q, S_k, H, D = 2, 6, 5, 3, 4
    for q_offset in (0, 1, -1):
        q = rng.standard_normal((B, S_q, H, D))
        k = rng.standard_normal((B, S_k, D))
        w = rng.standard_normal((B, S_q, H))
        key_of = dense_key_of(B, S_q, S_k, q_offset)
        I = rng.standard_normal((B, S_q, S_k))
        p = random_p(rng, key_of)
        d = oracle.Problem(q, k, w, I, p, None, q_offset=q_offset).backward()
        s = oracle.Problem(q, k, w, I, p, key_of.astype(np.int32), S_k=S_k).backward()
        for u, v in zip(d, s):
            np.testing.assert_allclose(u, v, rtol=1e-14, atol=1e-15)


def test_sampled_entry_points_match_full():
    """rows() and dk_rows() (used for full-size sampled parity) agree with the
    full backward."""
    x = make_inputs("tiny")
    prob = oracle.Problem.from_inputs(x)
    dq, dw, dk = prob.backward()
    rows = [0, 5, 17, 63]
    rq, rw = prob.rows(rows)
    assert np.array_equal(rq, dq[0, rows]) and np.array_equal(rw, dw[0, rows])
    keys = [0, 3, 64, 127]
    np.testing.assert_allclose(prob.dk_rows(keys), dk[0, keys], rtol=1e-12, atol=1e-14)
    xd = make_inputs("dense", S_q=16, seed=1)
    # dense inputs cut to 24 keys, 4 heads, 8 dims (rows t < 16 only see keys s <= t)
    small = oracle.Problem(oracle.widen_bf16(xd.q[:, :, :4, :8]), oracle.widen_bf16(xd.k[:, :24, :8]),
                           xd.w[:, :, :4], xd.index_score[:, :, :24], xd.attn_score[:, :, :24], None)
    dq, dw, dk = small.backward()
    rq, rw = small.rows([1, 15])
    assert np.array_equal(rq, dq[0, [1, 15]]) and np.array_equal(rw, dw[0, [1, 15]])
    np.testing.assert_allclose(small.dk_rows([0, 7, 23]), dk[0, [0, 7, 23]], rtol=1e-12, atol=1e-14)


def test_oracle_error_paths():
    x = make_inputs("tiny")
    prob = oracle.Problem.from_inputs(x)
    with pytest.raises(RuntimeError):
        prob.rows([64])
    with pytest.raises(RuntimeError):
        prob.dk_rows([-1])


def test_relrms_metric():
    assert relrms([1.0, 2.0], [1.0, 2.0]) == 0.0
    assert abs(relrms([1.0, 0.0], [0.0, 1.0]) - np.sqrt(2.0)) < 1e-15
