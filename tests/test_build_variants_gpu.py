"""Build variants must agree bit for bit (race detection by construction).

The library's kernels keep short buffer rings: the row kernel two K tiles,
four slot stages and two sign-word buffers; the range kernel three Q' tiles,
two key tables and four record stages (the slot-row route stages its dK rows
in a K tile of the ring).  The deep-buffer build
(IBWD_DEEP_BUFFERS, libdsa_indexer_bwd_deepbuf.so) keeps 4/8/4 and 4/4/8 of
them with the same copy schedule, so none of its buffers is reused within a
copy's window.  A buffer the library reused too early (a missing wait or
barrier) would change its results and not the variant's: every output of the
two builds must be equal bit for bit, d_k included (the summation order does
not depend on the ring depth).  Cases: full-size workloads (long query loops
per key range), duplicate ids (the range kernel's ordered fallback pass),
short and ragged rows, bf16 outputs, one head group (H <= 32) at D = 64, on
both deterministic dK routes where they differ.
"""
import dataclasses

import numpy as np
import pytest

from synth import WORKLOADS, make_inputs
from tests.test_parity_gpu import call, dev_inputs, host, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ibwd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_lightning_indexer_bwd_amd as m
    m.library()
    return m


def both_builds(ibwd, x, **kw):
    t = dev_inputs(x)
    a = call(ibwd, x, t, **kw)
    torch.cuda.synchronize()
    a = host(a)
    with ibwd.using_library(ibwd.DEEPBUF_LIB_PATH):
        b = call(ibwd, x, t, **kw)
        torch.cuda.synchronize()
        b = host(b)
    return a, b


def assert_same_bits(name, a, b):
    for what, u, v in zip(("d_q", "d_w", "d_k"), a, b):
        assert u.dtype == v.dtype and u.shape == v.shape
        same = np.array_equal(u.view(np.uint8), v.view(np.uint8))
        if not same:
            diff = np.flatnonzero(u.view(np.uint8) != v.view(np.uint8))
            pytest.fail(f"{name}: {what} differs between builds at {diff.size} bytes (first {diff[:5]})")
    log(f"{name}: library and deep-buffer build bitwise equal")


@pytest.mark.parametrize("name", ["anchor", "dense", "wide", "anchor-topk256"])
def test_full_size_workloads(ibwd, name):
    log(f"case: build variants, full-size {name}")
    x = make_inputs(dataclasses.replace(WORKLOADS["anchor"], topk=256) if name == "anchor-topk256" else name)
    assert_same_bits(name, *both_builds(ibwd, x))


@pytest.mark.parametrize("route", ["key_ranges", "slot_rows"])
def test_duplicate_ids(ibwd, route):
    """Rows that select keys two or three times: the range kernel adds the
    losing records in its ordered fallback pass."""
    log(f"case: build variants, duplicate ids route={route}")
    x = make_inputs("anchor", S_q=1024, seed=91)
    ids = x.ids.copy()
    ids[:, :, 1::9] = ids[:, :, 0::9][:, :, :ids[:, :, 1::9].shape[2]]
    ids[:, ::5, 2::9] = ids[:, ::5, 0::9][:, :, :ids[:, ::5, 2::9].shape[2]]
    x.ids = ids
    assert_same_bits(f"duplicates-{route}", *both_builds(ibwd, x, dk_route=route))


@pytest.mark.parametrize("route", ["key_ranges", "slot_rows"])
def test_short_ragged_rows(ibwd, route):
    """topk 128 at the anchor's shapes with row t keeping min(t/2 + 1, 128)
    slots (a -1 tail): many empty (query, range) pairs and short chunk loops."""
    log(f"case: build variants, short ragged rows route={route}")
    wl = dataclasses.replace(WORKLOADS["anchor"], S_q=2048, topk=128)
    x = make_inputs(wl, seed=92)
    ids = x.ids.copy()
    for t in range(ids.shape[1]):
        ids[:, t, min(t // 2 + 1, ids.shape[2]):] = -1
    x.ids = ids
    assert_same_bits(f"ragged-{route}", *both_builds(ibwd, x, dk_route=route))


def test_bf16_outputs(ibwd):
    log("case: build variants, bf16 outputs")
    x = make_inputs("anchor", S_q=2048, seed=93)
    assert_same_bits("bf16", *both_builds(ibwd, x, bf16_out=True))


@pytest.mark.parametrize("route", ["key_ranges", "slot_rows"])
def test_one_head_group(ibwd, route):
    """H = 32 (one wave per row in the row kernel) at D = 64."""
    log(f"case: build variants, H=32 D=64 route={route}")
    wl = dataclasses.replace(WORKLOADS["sparse"], H=32, D=64, S_q=2048)
    x = make_inputs(wl, seed=94)
    assert_same_bits(f"h32d64-{route}", *both_builds(ibwd, x, dk_route=route))
