"""More pins of the fp64 oracle against facts that do not come from its code.

* a scalar-loop backward written here from the definition (plain Python
  floats, its own bf16 decoding), compared with the oracle on the tiny
  workload to 1e-12: a dropped term, a transposed operand or a wrong index in
  either fails it;
* the bf16 widening against values the bf16 format fixes by hand;
* the forward scores at sampled query rows (``t_index``) under a causal
  offset, against brute force;
* dK of sampled keys (``dk_rows``) against the full backward on rows that
  select some keys several times.

Definition followed: NVIDIA/cudnn-frontend PR #730, posted benchmark harness
(the fp64 `ref_grads` reference, the kernel-1 score-gradient contract, the
padding battery); duplicates are independent slots, padding contributes nothing.
"""
import math

import numpy as np

import oracle
from synth import make_inputs


def bf16_value(bits: int) -> float:
    """The real number a bf16 bit pattern encodes, from sign, exponent and
    fraction fields (IEEE binary16 'brain' layout: 1 + 8 + 7 bits)."""
    sign = -1.0 if bits & 0x8000 else 1.0
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0xFF:
        return sign * math.inf if frac == 0 else math.nan
    if exp == 0:
        return sign * math.ldexp(frac, -133)          # subnormal: frac * 2^(1-127-7)
    return sign * math.ldexp(128 + frac, exp - 134)   # (1 + frac/128) * 2^(exp-127)


def scalar_backward(q, k, w, ids, I, p, S_k, sm_scale, grad_loss):
    """dq, dw, dk by plain loops over query, slot, head and dimension.

    V = {j : 0 <= id_j < S_k};  P = softmax over V of sm_scale*I;
    dI_j = grad_loss*sm_scale*(P_j - p_j);  S = q.k;  G = dI*w*[S > 0];
    dW = sum_j dI_j*relu(S);  dQ = sum_j G*k;  dK[id_j] += sum_h G*q.
    """
    B, S_q, H, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    topk = len(ids[0][0])
    dq = [[[[0.0] * D for _ in range(H)] for _ in range(S_q)] for _ in range(B)]
    dw = [[[0.0] * H for _ in range(S_q)] for _ in range(B)]
    dk = [[[0.0] * D for _ in range(S_k)] for _ in range(B)]
    for b in range(B):
        for t in range(S_q):
            valid = [j for j in range(topk) if 0 <= ids[b][t][j] < S_k]
            if not valid:
                continue
            z = {j: sm_scale * I[b][t][j] for j in valid}
            zmax = max(z.values())
            den = sum(math.exp(z[j] - zmax) for j in valid)
            for j in valid:
                dI = grad_loss * sm_scale * (math.exp(z[j] - zmax) / den - p[b][t][j])
                s = ids[b][t][j]
                for h in range(H):
                    S = 0.0
                    for d in range(D):
                        S += q[b][t][h][d] * k[b][s][d]
                    if S > 0.0:
                        dw[b][t][h] += dI * S
                        g = dI * w[b][t][h]
                        for d in range(D):
                            dq[b][t][h][d] += g * k[b][s][d]
                            dk[b][s][d] += g * q[b][t][h][d]
    return np.array(dq), np.array(dw), np.array(dk)


def test_scalar_loop_backward_matches_oracle_tiny():
    """The tiny workload (B=1, H=4, D=32, S_q=64, S_k=128, topk=16, ~10% padding,
    garbage index/attn scores on padded slots), sm_scale 0.9, grad_loss 1.3."""
    x = make_inputs("tiny")
    S_k = x.wl.S_k
    q = [[[[bf16_value(int(v)) for v in hd] for hd in th] for th in bt] for bt in x.q]
    k = [[[bf16_value(int(v)) for v in sd] for sd in bs] for bs in x.k]
    w = x.w.astype(np.float64).tolist()
    I = x.index_score.astype(np.float64).tolist()
    p = x.attn_score.astype(np.float64).tolist()
    ids = x.ids.tolist()
    ref = scalar_backward(q, k, w, ids, I, p, S_k, 0.9, 1.3)
    prob = oracle.Problem.from_inputs(x)
    prob.sm_scale, prob.grad_loss = 0.9, 1.3
    got = prob.backward()
    for name, g, r in zip(("dq", "dw", "dk"), got, ref):
        scale = np.abs(r).max()
        assert scale > 0, name
        err = np.abs(g - r).max() / scale
        assert err <= 1e-12, f"{name}: {err:.3e}"


def test_widen_bf16_hand_values():
    """Bit patterns whose values the bf16 format fixes: one, signed zero, the
    smallest and largest subnormal, the smallest normal, the largest finite
    value, an exact small integer, infinities."""
    cases = {
        0x3F80: 1.0,
        0xBF80: -1.0,
        0x0000: 0.0,
        0x8000: -0.0,
        0x0001: 2.0 ** -133,
        0x007F: 127 * 2.0 ** -133,
        0x0080: 2.0 ** -126,
        0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,
        0x42F7: 123.5,
        0xC2F7: -123.5,
        0x4049: 3.140625,
        0x7F80: math.inf,
        0xFF80: -math.inf,
    }
    bits = np.array(list(cases), dtype=np.uint16)
    got = oracle.widen_bf16(bits)
    assert got.dtype == np.float64
    for b, g in zip(bits, got):
        want = cases[int(b)]
        assert g == want and math.copysign(1.0, g) == math.copysign(1.0, want), hex(b)
        assert bf16_value(int(b)) == want
    # the decoder above and the oracle agree on every finite pattern
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (allb >> 7) & 0xFF
    fin = allb[exp != 0xFF]
    wid = oracle.widen_bf16(fin)
    ref = np.array([bf16_value(int(b)) for b in fin])
    assert np.array_equal(wid, ref)


def test_forward_scores_sampled_rows_causal():
    """forward_scores on rows of q and w that are query rows t_index of a longer
    sequence: the causal mask uses t_index, not the row position."""
    rng = np.random.default_rng(17)
    B, S_q, S_k, H, D = 1, 12, 10, 3, 5
    q = rng.standard_normal((B, S_q, H, D))
    k = rng.standard_normal((B, S_k, D))
    w = rng.standard_normal((B, S_q, H))
    rows = np.array([0, 3, 7, 11])
    for off in (0, -2, 3):
        got = oracle.forward_scores(q[:, rows], k, w[:, rows], off, rows)
        for i, t in enumerate(rows):
            for s in range(S_k):
                if s > t + off:
                    assert got[0, i, s] == -np.inf
                    continue
                tot = 0.0
                for h in range(H):
                    dot = sum(q[0, t, h, d] * k[0, s, d] for d in range(D))
                    tot += w[0, t, h] * max(dot, 0.0)
                assert abs(got[0, i, s] - tot) <= 1e-12 * max(1.0, abs(tot))


def test_dk_rows_with_duplicate_ids_match_full():
    """dk_rows (used for sampled full-size parity) equals the full backward's dK
    when rows select some keys two or three times."""
    x = make_inputs("tiny", seed=77)
    ids = x.ids.copy()
    ids[0, :, 1] = ids[0, :, 0]          # every row repeats its first key
    ids[0, ::3, 2] = ids[0, ::3, 0]      # every third row: three times
    ids[0, 5, :] = 9                     # one row of a single key
    x.ids = ids
    prob = oracle.Problem.from_inputs(x)
    _, _, dk = prob.backward()
    keys = np.unique(np.concatenate([ids[0, :, 0][ids[0, :, 0] >= 0], [9, 0, 127]]))
    got = prob.dk_rows(keys)
    np.testing.assert_allclose(got, dk[0, keys], rtol=1e-12, atol=1e-14)
    # a repeated slot counts twice: removing the repeat changes dK of that key
    x2 = make_inputs("tiny", seed=77)
    d2 = oracle.Problem.from_inputs(x2).backward()[2]
    assert np.abs(d2[0, 9] - dk[0, 9]).max() > 0
