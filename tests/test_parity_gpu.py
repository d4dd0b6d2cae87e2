"""GPU parity of the HIP path against the fp64 oracle (through the C ABI).

Bars (relative RMS = ||a-b||/||b||, the PR #730 harness metric):
  d_index_q, d_weights: relRMS <= 2e-3 and max|a-b| <= 1e-2 * max|ref|
  d_index_k (fp32 atomics, any summation order): relRMS <= 5e-3
d_q and d_w are also bitwise reproducible run to run; padding slots (-1,
other negatives, positive out-of-range) are bitwise equivalent for d_q/d_w
(analogue of the PR #730 padding battery).
"""
import dataclasses

import numpy as np
import pytest

import oracle
from synth import WORKLOADS, make_inputs
from tests.util import bf16_bits_to_f32, bf16_rne_bits, maxabs, relrms

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DQ_DW_REL = 2e-3
DQ_DW_MAXABS = 1e-2
DK_REL = 5e-3
# unit roundoff of bf16 (8 significant bits)
BF16_U = 2.0 ** -8


@pytest.fixture(scope="module")
def ibwd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_lightning_indexer_bwd_amd as m
    m.library()
    return m


def log(msg):
    print(msg, flush=True)


def dev_inputs(x):
    d = torch.device("cuda:0")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(d)

    out = dict(q=bf16(x.q), k=bf16(x.k), w=torch.from_numpy(x.w).to(d),
               I=torch.from_numpy(x.index_score).to(d), p=torch.from_numpy(x.attn_score).to(d))
    out["ids"] = None if x.ids is None else torch.from_numpy(x.ids).to(d)
    return out


def call(ibwd, x, t, outs=(None, None, None), **kw):
    """Enqueue one library call on the current stream (no synchronisation)."""
    if x.ids is None:
        return ibwd.indexer_bwd_dense(t["q"], t["k"], t["w"], t["I"], t["p"], *outs,
                                      q_offset=x.wl.q_offset, sm_scale=x.sm_scale,
                                      grad_loss=x.grad_loss, **kw)
    return ibwd.indexer_bwd_sparse(t["q"], t["k"], t["w"], t["ids"], t["I"], t["p"], *outs,
                                   sm_scale=x.sm_scale, grad_loss=x.grad_loss, **kw)


def host(r):
    """Outputs as numpy: fp32 values, bf16 as their uint16 bit patterns."""
    return [a.view(torch.int16).cpu().numpy().view(np.uint16) if a.dtype == torch.bfloat16
            else a.cpu().numpy() for a in r]


def run(ibwd, x, t=None, deterministic=False, atomic_dk=False, bf16_out=False, dk_route="auto"):
    t = dev_inputs(x) if t is None else t
    kw = {} if dk_route == "auto" else dict(dk_route=dk_route)
    r = call(ibwd, x, t, deterministic=deterministic, atomic_dk=atomic_dk, bf16_out=bf16_out, **kw)
    torch.cuda.synchronize()
    return host(r)


def assert_parity(name, got, ref):
    """The bars above, for fp32 and bf16 outputs alike."""
    dq, dw, dk = got
    rq, rw, rk = ref
    e = dict(dq=relrms(dq, rq), dw=relrms(dw, rw), dk=relrms(dk, rk),
             dq_max=maxabs(dq, rq) / max(np.abs(rq).max(), 1e-30),
             dw_max=maxabs(dw, rw) / max(np.abs(rw).max(), 1e-30))
    log(f"{name}: " + " ".join(f"{k}={v:.3e}" for k, v in e.items()))
    for a in (dq, dw, dk):
        assert np.isfinite(a).all()

    assert e["dq"] <= DQ_DW_REL and e["dq_max"] <= DQ_DW_MAXABS, e
    assert e["dw"] <= DQ_DW_REL and e["dw_max"] <= DQ_DW_MAXABS, e
    assert e["dk"] <= DK_REL, e
    return e


def small(name, S_q, **kw):
    wl = dataclasses.replace(WORKLOADS[name], S_q=S_q, **kw)
    return wl


# ---------------------------------------------------------------------------
# full comparison at sizes the oracle finishes in seconds

def test_tiny_workload(ibwd):
    log("case: tiny workload, full oracle")
    x = make_inputs("tiny")
    assert_parity("tiny", run(ibwd, x), oracle.Problem.from_inputs(x).backward())


@pytest.mark.parametrize("name,S_q", [("sparse", 96), ("anchor", 64), ("wide", 40), ("dense", 200)])
def test_workload_shapes_reduced_queries(ibwd, name, S_q):
    """The real H, D, S_k, topk (and id structure) of each workload, fewer queries."""
    log(f"case: {name} S_q={S_q}, full oracle")
    x = make_inputs(name, S_q=S_q, seed=100 + S_q)
    assert_parity(f"{name}-Sq{S_q}", run(ibwd, x), oracle.Problem.from_inputs(x).backward())


ROUTES = ["key_ranges", "slot_rows"]


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("topk,H,D,pad", [(1, 4, 32, 0.0), (37, 64, 128, 0.1), (100, 33, 64, 0.3),
                                          (129, 1, 32, 0.05), (300, 64, 64, 0.5), (16, 17, 128, 1.0),
                                          (70, 32, 128, 0.2), (1000, 8, 32, 0.2), (1024, 64, 128, 0.1),
                                          (1025, 64, 64, 0.1)])
def test_ragged_and_odd_shapes(ibwd, topk, H, D, pad, route):
    """topk not a multiple of any chunk, H below/above MFMA tiles, every D, heavy
    padding, an all-padding workload; both deterministic dK routes.  1000, 1024
    and 1025 sit at the prep kernel's limit for keeping its range masks in
    registers (rows of at most 1024 slots; longer rows take the other build)."""
    log(f"case: ragged topk={topk} H={H} D={D} pad={pad} route={route}")
    wl = dataclasses.replace(WORKLOADS["tiny"], H=H, D=D, S_q=48, S_k=max(160, topk + 1), topk=topk,
                             pad_frac=pad)
    x = make_inputs(wl, seed=7 + topk)
    got = run(ibwd, x, dk_route=route)
    ref = oracle.Problem.from_inputs(x).backward()
    if pad >= 1.0:
        assert all(np.all(a == 0) for a in got)
        return
    assert_parity(f"ragged-{topk}-{H}-{D}-{route}", got, ref)


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("S_k,topk", [(40000, 700), (262144, 300)])
def test_many_key_ranges(ibwd, S_k, topk, route):
    """More than 64 key ranges of 128 keys (313, and 2048 at the largest S_k the
    library accepts): the range scan with several ranges per lane, range ids of
    up to 11 bits in the ballot ranking, and many range (or key-block) workgroups."""
    log(f"case: many ranges S_k={S_k} topk={topk} route={route}")
    wl = dataclasses.replace(WORKLOADS["tiny"], H=8, D=32, S_q=24, S_k=S_k, topk=topk, pad_frac=0.05)
    x = make_inputs(wl, seed=S_k % 1000 + topk)
    assert_parity(f"ranges-{S_k}-{topk}-{route}", run(ibwd, x, dk_route=route),
                  oracle.Problem.from_inputs(x).backward())


def test_batches_local_ids_do_not_alias(ibwd):
    """B=2: positive out-of-range ids of batch 0 are padding, not keys of batch 1."""
    log("case: B=2 local ids")
    wl = dataclasses.replace(WORKLOADS["tiny"], B=2, S_q=40, pad_frac=0.2)
    x = make_inputs(wl, seed=21)
    pad = x.ids < 0
    n = np.arange(x.ids.size).reshape(x.ids.shape)
    x.ids[pad] = wl.S_k + (n[pad] % 5)
    assert_parity("B2", run(ibwd, x), oracle.Problem.from_inputs(x).backward())


@pytest.mark.parametrize("sm_scale,grad_loss", [(1.0, 0.5), (1.0, 1.5), (0.35, 1.0), (2.0, -1.0)])
def test_scalars(ibwd, sm_scale, grad_loss):
    log(f"case: sm_scale={sm_scale} grad_loss={grad_loss}")
    x = make_inputs("anchor", S_q=32, seed=5, sm_scale=sm_scale, grad_loss=grad_loss)
    assert_parity(f"scalars-{sm_scale}-{grad_loss}", run(ibwd, x), oracle.Problem.from_inputs(x).backward())


@pytest.mark.parametrize("q_offset", [0, -3, 5, -70])
def test_dense_q_offset(ibwd, q_offset):
    log(f"case: dense q_offset={q_offset}")
    wl = dataclasses.replace(WORKLOADS["dense"], S_q=64, S_k=96, q_offset=q_offset)
    x = make_inputs(wl, seed=3)
    got = run(ibwd, x)
    ref = oracle.Problem.from_inputs(x).backward()
    if q_offset <= -64:
        assert all(np.all(a == 0) for a in got)
        return
    assert_parity(f"dense-off{q_offset}", got, ref)

@pytest.mark.parametrize("atomic_dk,route", [(False, "key_ranges"), (False, "slot_rows"), (True, "auto")])
def test_global_ids(ibwd, atomic_dk, route):
    """B=3 with global ids (key id - b*S_k of batch b): the valid slots of the
    local-id case shifted by b*S_k, and its padding slots replaced by keys of
    the other batches, ids past B*S_k and negatives.  Equal to the local-id
    call (bitwise on the default route) and to the oracle on the remapped ids."""
    log(f"case: B=3 global ids atomic={atomic_dk} route={route}")
    wl = dataclasses.replace(WORKLOADS["tiny"], B=3, S_q=40, S_k=300, topk=96, pad_frac=0.3)
    x = make_inputs(wl, seed=41)
    S_k = wl.S_k
    base = (np.arange(wl.B, dtype=np.int64) * S_k)[:, None, None]
    pad = x.ids < 0
    n = np.arange(x.ids.size).reshape(x.ids.shape)
    other = (base + S_k * (1 + n % (wl.B - 1)) + n % S_k) % (wl.B * S_k)   # another batch's key
    junk = np.where(n % 3 == 0, other, np.where(n % 3 == 1, wl.B * S_k + n % 7, -1 - n % 4))
    g = np.where(pad, junk, x.ids + base).astype(np.int32)
    local = oracle.global_ids_to_local(g, S_k)
    assert np.array_equal(local, np.where(pad, -1, x.ids))
    t = dev_inputs(x)
    ref_local = run(ibwd, x, t, atomic_dk=atomic_dk, dk_route=route)
    tg = dict(t, ids=torch.from_numpy(g).to(t["q"].device))
    got = ibwd.indexer_bwd_sparse(tg["q"], tg["k"], tg["w"], tg["ids"], tg["I"], tg["p"],
                                  sm_scale=x.sm_scale, grad_loss=x.grad_loss, atomic_dk=atomic_dk,
                                  global_ids=True, dk_route=route)
    torch.cuda.synchronize()
    got = [a.cpu().numpy() for a in got]
    assert np.array_equal(got[0], ref_local[0]) and np.array_equal(got[1], ref_local[1])
    if atomic_dk:
        assert relrms(got[2], ref_local[2]) < 1e-5
    else:
        assert np.array_equal(got[2], ref_local[2])
    x.ids = local
    assert_parity(f"global-atomic{int(atomic_dk)}-{route}", got, oracle.Problem.from_inputs(x).backward())


@pytest.mark.parametrize("name,S_q,topk", [("tiny", 64, 0), ("anchor", 192, 0), ("dense", 160, 0),
                                           ("anchor", 192, 128)])
def test_bf16_outputs(ibwd, name, S_q, topk):
    """bf16 outputs within the same bars as fp32 outputs (not widened): d_w and
    d_k are the fp32 outputs of the same call rounded to nearest even, bit for
    bit; d_q is rounded from a dQ whose G' enters GEMM2 as two bf16 terms.
    topk 128 of 4096 keys takes the slot-row dK route."""
    log(f"case: bf16 outputs {name} S_q={S_q} topk={topk}")
    wl = dataclasses.replace(WORKLOADS[name], S_q=S_q, **({"topk": topk} if topk else {}))
    x = make_inputs(wl, seed=51)
    t = dev_inputs(x)
    f32 = run(ibwd, x, t)
    b16 = run(ibwd, x, t, bf16_out=True)
    for a in b16:
        assert a.dtype == np.uint16
    assert np.array_equal(b16[1], bf16_rne_bits(f32[1]))
    assert np.array_equal(b16[2], bf16_rne_bits(f32[2]))
    ref = oracle.Problem.from_inputs(x).backward()
    e = assert_parity(f"bf16-{name}-{topk}", [bf16_bits_to_f32(b) for b in b16], ref)
    # every d_q element is the oracle's value up to one rounding to bf16 (half a
    # unit in the last place, 2^-8 relative) and fp32 accumulation error: the
    # G' of its product lost nothing to bf16
    dq = bf16_bits_to_f32(b16[0]).astype(np.float64)
    rq = ref[0]
    slack = 1e-5 * np.abs(rq).max()
    assert np.all(np.abs(dq - rq) <= BF16_U * np.abs(rq) + slack), np.max(
        np.abs(dq - rq) - BF16_U * np.abs(rq))


@pytest.mark.parametrize("bf16_out,topk", [(False, 1024), (True, 1024), (False, 128)])
def test_graph_capture_replays(ibwd, bf16_out, topk):
    """The call captured in a HIP graph (the library enqueues kernels only, no
    allocation, memset or host synchronisation): every replay, with eager
    library calls on other inputs and synchronisations in between, is bitwise
    equal to the eager call."""
    log(f"case: graph capture bf16_out={bf16_out} topk={topk}")
    wl = dataclasses.replace(WORKLOADS["anchor"], topk=topk)
    x = make_inputs(wl, S_q=256, seed=61)
    y = make_inputs(wl, S_q=256, seed=62)
    tx, ty = dev_inputs(x), dev_inputs(y)
    ref = run(ibwd, x, tx, bf16_out=bf16_out)
    dt = torch.bfloat16 if bf16_out else torch.float32
    B, S_q, H, D = tx["q"].shape
    S_k = tx["k"].shape[1]
    outs = (torch.empty((B, S_q, H, D), dtype=dt, device="cuda:0"),
            torch.empty((B, S_q, H), dtype=dt, device="cuda:0"),
            torch.empty((B, S_k, D), dtype=dt, device="cuda:0"))
    ws_bytes = ibwd.indexer_bwd_workspace_bytes(False, B, S_q, S_k, H, D, tx["ids"].shape[-1], 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm-up on the capture stream
        call(ibwd, x, tx, outs, bf16_out=bf16_out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(ibwd, x, tx, outs, bf16_out=bf16_out, workspace=ws)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        other = run(ibwd, y, ty, bf16_out=bf16_out)   # eager work on other inputs
        assert not np.array_equal(other[0], ref[0])
        g.replay()
        torch.cuda.synchronize()
        for u, v in zip(host(outs), ref):
            assert np.array_equal(u, v), rep
    del g


# ---------------------------------------------------------------------------
# padding equivalence and determinism

def test_padding_equivalence(ibwd):
    log("case: padding equivalence")
    x = make_inputs("anchor", S_q=128, seed=9, pad_frac=0.2)
    base = run(ibwd, x)
    pad = x.ids == -1
    n = np.arange(x.ids.size).reshape(x.ids.shape)
    x.ids[pad] = np.where(n[pad] % 2 == 0, x.wl.S_k + (n[pad] % 9999), -5)
    x.index_score[pad] = 3.0e3
    x.attn_score[pad] = 0.777
    alt = run(ibwd, x)
    assert np.array_equal(base[0], alt[0]) and np.array_equal(base[1], alt[1])
    assert relrms(alt[2], base[2]) < 1e-6


@pytest.mark.parametrize("topk", [1024, 128])
def test_run_to_run_bitwise(ibwd, topk):
    """Both deterministic routes (the key-range route at topk 1024, the slot-row
    route at 128 of 4096 keys) are bitwise reproducible for all three outputs;
    d_q and d_w do not depend on the route."""
    log(f"case: run-to-run determinism topk={topk}")
    wl = dataclasses.replace(WORKLOADS["anchor"], topk=topk)
    x = make_inputs(wl, S_q=256, seed=13)
    t = dev_inputs(x)
    a = run(ibwd, x, t)
    b = run(ibwd, x, t, deterministic=True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    other = run(ibwd, x, t, dk_route="key_ranges" if topk == 128 else "slot_rows")
    assert np.array_equal(other[0], a[0]) and np.array_equal(other[1], a[1])


@pytest.mark.parametrize("name", ["tiny", "anchor", "dense"])
def test_atomic_route(ibwd, name):
    """The single-pass fp32-atomic dK route: parity, and d_q/d_w bitwise run to run."""
    log(f"case: atomic route {name}")
    x = make_inputs(name, S_q=min(WORKLOADS[name].S_q, 96), seed=23)
    t = dev_inputs(x)
    a = run(ibwd, x, t, atomic_dk=True)
    b = run(ibwd, x, t, atomic_dk=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert relrms(a[2], b[2]) < 1e-5
    assert_parity(f"atomic-{name}", a, oracle.Problem.from_inputs(x).backward())
    d = run(ibwd, x, t)
    assert np.array_equal(a[0], d[0]) and np.array_equal(a[1], d[1])


@pytest.mark.parametrize("atomic_dk,route", [(False, "key_ranges"), (False, "slot_rows"), (True, "auto")])
@pytest.mark.parametrize("S_k,topk", [(300, 200), (4096, 96)])
def test_duplicate_ids(ibwd, atomic_dk, route, S_k, topk):
    """Duplicate ids in a row are independent slots (both routes; the default
    route's range kernel takes its ordered path for tiles with repeated keys).
    At 96 of 4096 keys the range kernel's waves also pass over key blocks
    without a record of the query."""
    log(f"case: duplicate ids atomic={atomic_dk} route={route} S_k={S_k} topk={topk}")
    wl = dataclasses.replace(WORKLOADS["anchor"], S_q=48, S_k=S_k, topk=topk, pad_frac=0.05)
    x = make_inputs(wl, seed=31 + topk)
    rng = np.random.default_rng(5)
    # every row: a third of its slots repeat keys of the row (some several times)
    for t in range(wl.S_q):
        src = rng.integers(0, wl.topk, size=wl.topk // 3)
        dst = rng.integers(0, wl.topk, size=wl.topk // 3)
        x.ids[0, t, dst] = x.ids[0, t, src]
    x.ids[0, 0, :] = 7          # a row of one key repeated
    got = run(ibwd, x, atomic_dk=atomic_dk, dk_route=route)
    assert_parity(f"dup-atomic{int(atomic_dk)}-{route}-{S_k}", got, oracle.Problem.from_inputs(x).backward())


@pytest.mark.parametrize("route", ROUTES)
def test_ragged_row_lengths(ibwd, route):
    """Per-row valid lengths that ramp up with the query (row t keeps its first
    min(t//2 + 1, topk) slots, the rest are -1), at the anchor's H, D, S_k and
    topk: every chunk count from 1 to the full row, a partial last chunk."""
    log(f"case: ragged row-length ramp route={route}")
    wl = dataclasses.replace(WORKLOADS["anchor"], S_q=2048, pad_frac=0.0)
    x = make_inputs(wl, seed=51)
    t = np.arange(wl.S_q)[:, None]
    j = np.arange(wl.topk)[None, :]
    x.ids[0][j >= np.minimum(t // 2 + 1, wl.topk)] = -1
    assert_parity(f"ramp-{route}", run(ibwd, x, dk_route=route), oracle.Problem.from_inputs(x).backward())


@pytest.mark.parametrize("pad", [0.0, 0.4])
def test_one_full_key_range(ibwd, pad):
    """Every valid id of a row in the first 128-key range: that range holds all
    the row's records (128 without padding, the range kernel's staged record
    block exactly full) and the other ranges none."""
    log(f"case: one full key range pad={pad}")
    wl = dataclasses.replace(WORKLOADS["anchor"], S_q=40, S_k=512, topk=128, pad_frac=0.0)
    x = make_inputs(wl, seed=41)
    rng = np.random.default_rng(9)
    for t in range(wl.S_q):
        x.ids[0, t] = rng.permutation(128)
    if pad:
        x.ids[rng.random(x.ids.shape) < pad] = -1
    assert_parity(f"full-range-{pad}", run(ibwd, x), oracle.Problem.from_inputs(x).backward())


def test_inputs_are_not_modified(ibwd):
    log("case: inputs read-only")
    x = make_inputs("tiny")
    t = dev_inputs(x)
    before = {k: v.clone() for k, v in t.items() if v is not None}
    run(ibwd, x, t)
    for k, v in before.items():
        assert torch.equal(v, t[k]), k


def test_invalid_call_leaves_outputs_untouched(ibwd):
    log("case: invalid call")
    x = make_inputs("tiny")
    t = dev_inputs(x)
    dq = torch.full((1, 64, 4, 32), 7.0, device="cuda:0")
    dw = torch.full((1, 64, 4), 7.0, device="cuda:0")
    dk = torch.full((1, 128, 32), 7.0, device="cuda:0")
    lib = ibwd.library()
    st = lib.indexer_bwd_sparse(t["q"].data_ptr(), t["k"].data_ptr(), t["w"].data_ptr(),
                                t["ids"].data_ptr(), t["I"].data_ptr(), t["p"].data_ptr(),
                                dq.data_ptr(), dw.data_ptr(), dk.data_ptr(), 1, 64, 128, 4, 40, 16,
                                1.0, 1.0, 0, None, 0, None)
    torch.cuda.synchronize()
    assert st == ibwd.IBWD_ERR_INVALID_ARGUMENT
    assert bool((dq == 7).all() and (dw == 7).all() and (dk == 7).all())


# ---------------------------------------------------------------------------
# full-size workloads, in the configuration the benchmark times: every element
# of d_q, d_w and d_k against the full oracle backward (seconds on the host
# cores)

@pytest.mark.parametrize("name", ["sparse", "anchor", "wide", "dense", "anchor-topk128", "sparse-key-ranges"])
def test_full_size_workload(ibwd, name):
    """The four workloads (sparse, at 512 of 4096 keys, on the slot-row dK route
    by density), the anchor at topk 128, and the sparse workload on the key-range
    route."""
    log(f"case: full-size {name}")
    wl = dataclasses.replace(WORKLOADS["anchor"], topk=128) if name == "anchor-topk128" else \
        "sparse" if name == "sparse-key-ranges" else name
    x = make_inputs(wl, device="cuda:0")
    got = run(ibwd, x, dk_route="key_ranges" if name == "sparse-key-ranges" else "auto")
    ref = oracle.Problem.from_inputs(x).backward()
    assert_parity(f"full-{name}", got, ref)
    # Euler identity of the 1-homogeneous score at every (t,h): <q, dQ> = w dW
    q = oracle.widen_bf16(x.q)
    lhs = np.einsum("bthd,bthd->bth", q, got[0].astype(np.float64))
    rhs = x.w.astype(np.float64) * got[1].astype(np.float64)
    e = relrms(lhs, rhs)
    log(f"full-{name}: euler relRMS {e:.3e}")
    assert e < 6e-3, e


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("topk", [128, 256, 384, 640, 1536])
def test_topk_sweep_anchor_shapes(ibwd, topk, route):
    """The topk sweep points at the anchor's H, D and S_k (256 queries, 2%
    padding), on both deterministic dK routes: every element against the oracle."""
    log(f"case: topk sweep {topk} route={route}")
    wl = dataclasses.replace(WORKLOADS["anchor"], S_q=256, topk=topk)
    x = make_inputs(wl, seed=300 + topk)
    assert_parity(f"topk-{topk}-{route}", run(ibwd, x, dk_route=route),
                  oracle.Problem.from_inputs(x).backward())


def test_side_stream_without_workspace(ibwd):
    """A call on a side stream with no workspace, followed at once by
    allocations and fills on the current stream: the workspace the binding
    allocates belongs to the side stream, so that work cannot take its memory
    while the kernels run.  The outputs equal those of a plain call."""
    log("case: side stream, binding-allocated workspace")
    x = make_inputs("anchor", S_q=512, seed=71)
    t = dev_inputs(x)
    ref = run(ibwd, x, t)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    r = call(ibwd, x, t, stream=s)
    junk = [torch.full((1 << 22,), float(i), device="cuda:0") for i in range(16)]
    torch.cuda.synchronize()
    for u, v in zip(host(r), ref):
        assert np.array_equal(u, v)
    del junk


def test_stage_hook_reports_every_kernel(ibwd):
    """The profiling hook runs once per enqueued kernel, in launch order, on both routes."""
    log("case: stage hook")
    x = make_inputs("tiny", seed=3)
    y = make_inputs(dataclasses.replace(WORKLOADS["anchor"], S_q=64, topk=128), seed=3)
    seen = []
    ibwd.set_stage_hook(lambda stage, name: seen.append((stage, name)))
    try:
        a = run(ibwd, x, dk_route="key_ranges")
        b = run(ibwd, x, atomic_dk=True)
        run(ibwd, y)  # 128 of 4096 keys: the slot-row route by density
    finally:
        ibwd.set_stage_hook(None)
    assert seen == [(0, "row_prep_kernel"), (1, "row_export_kernel"), (2, "dk_range_kernel"),
                    (3, "dk_sum_kernel"), (0, "zero_u32_kernel"), (1, "row_kernel"),
                    (0, "row_prep_kernel"), (1, "row_export_kernel"), (2, "dk_rows_kernel"),
                    (3, "dk_sum_kernel")]
    c = run(ibwd, x, dk_route="key_ranges")  # hook removed: nothing more is reported
    assert len(seen) == 10
    assert all(np.array_equal(u, v) for u, v in zip(a, c))
    assert_parity("hook-atomic", b, oracle.Problem.from_inputs(x).backward())
