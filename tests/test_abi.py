"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and rejects invalid arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import dsa_lightning_indexer_bwd_amd as ibwd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_indexer_bwd.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(indexer_bwd_\w+)\s*\(", src)))


@pytest.mark.parametrize("path", [ibwd.LIB_PATH, ibwd.DEEPBUF_LIB_PATH])
def test_library_exports_every_declared_symbol(path):
    """The library and its deep-buffer build (the verification variant)."""
    names = declared_functions()
    assert set(names) >= {"indexer_bwd_sparse", "indexer_bwd_dense", "indexer_bwd_workspace_bytes",
                          "indexer_bwd_strerror"}
    lib = ctypes.CDLL(path)
    for n in names:
        assert hasattr(lib, n), n


def test_using_library_switches_and_restores():
    main = ibwd.library()
    with ibwd.using_library(ibwd.DEEPBUF_LIB_PATH) as deep:
        assert ibwd.library() is deep and deep is not main
        # host-side logic is the same in both builds
        assert ibwd.indexer_bwd_workspace_bytes(False, 1, 8192, 4096, 64, 128, 1024, 0) == \
            main.indexer_bwd_workspace_bytes(0, 1, 8192, 4096, 64, 128, 1024, 0)
    assert ibwd.library() is main
    with pytest.raises(RuntimeError):
        with ibwd.using_library("/nonexistent/libdsa_indexer_bwd.so"):
            pass
    assert ibwd.library() is main


def test_strerror_and_workspace():
    for st in (0, -1, -2, -3, 7):
        assert isinstance(ibwd.indexer_bwd_strerror(st), str)
    # default (two-pass) route: 16-byte slot records, (w*q)^T in bf16, dK partial slabs
    ws = ibwd.indexer_bwd_workspace_bytes(False, 1, 8192, 4096, 64, 128, 1024, 0)
    assert ws >= 8192 * 1024 * 16 + 8192 * 64 * 128 * 2 + 4096 * 128 * 4
    assert ws == ibwd.indexer_bwd_workspace_bytes(False, 1, 8192, 4096, 64, 128, 1024,
                                                  ibwd.IBWD_FLAG_DETERMINISTIC)
    assert ibwd.indexer_bwd_workspace_bytes(False, 1, 8192, 4096, 64, 128, 1024,
                                            ibwd.IBWD_FLAG_ATOMIC_DK) == 0
    assert ibwd.indexer_bwd_workspace_bytes(True, 2, 64, 64, 4, 32, 0, 0) >= 2 * 64 * 64 * 16
    assert ibwd.indexer_bwd_workspace_bytes(False, 0, 1, 1, 1, 32, 1, 0) == 0
    assert ibwd.indexer_bwd_workspace_bytes(False, 1, 1, 1, 1, 48, 1, 0) == 0
    assert ibwd.indexer_bwd_workspace_bytes(False, 1, 64, 128, 4, 32, 129, 0) == 0   # topk > S_k


def test_dk_route_flags_and_workspace():
    """The deterministic dK route follows the selection density (slot rows when
    topk*8 <= S_k) unless a flag forces one; the workspace follows the route."""
    KR, SR = ibwd.IBWD_FLAG_DK_KEY_RANGES, ibwd.IBWD_FLAG_DK_SLOT_ROWS
    wsb = ibwd.indexer_bwd_workspace_bytes
    rows, NR, NQB = 8192, 32, 16
    for topk, auto_rows in ((128, True), (512, True), (513, False), (1024, False)):
        auto = wsb(False, 1, 8192, 4096, 64, 128, topk, 0)
        kr = wsb(False, 1, 8192, 4096, 64, 128, topk, KR)
        sr = wsb(False, 1, 8192, 4096, 64, 128, topk, SR)
        assert auto == (sr if auto_rows else kr)
        assert kr != sr
        # slot rows: {position, dI} and a key per slot, a bf16 dK row per slot plus
        # one, the range table, the per query-block slabs
        slot_rows_bytes = (rows * topk * (8 + 4) + (rows * topk + 1) * 128 * 2 + rows * NR * 8
                           + NQB * NR * 128 * 128 * 4)
        assert slot_rows_bytes <= sr <= slot_rows_bytes + 5 * 256
    # rows past 4 GiB: the density rule falls back to key ranges, the forced route is refused
    big = (1, 8192, 1 << 18, 64, 128, 2048)      # 8192*2048 slots of 256-byte rows = 4 GiB
    assert wsb(False, *big, SR) == 0
    assert wsb(False, *big, 0) == wsb(False, *big, KR) > 0
    assert call_sparse(sparse_args(S_q=8192, S_k=1 << 18, H=64, D=128, topk=2048, flags=SR,
                                   ws_bytes=1 << 40)) == ibwd.IBWD_ERR_INVALID_ARGUMENT
    # the dense call always takes the key ranges: the slot-row flag is an error there
    assert wsb(True, 1, 64, 64, 4, 32, 0, SR) == 0
    assert wsb(True, 1, 64, 64, 4, 32, 0, KR) == wsb(True, 1, 64, 64, 4, 32, 0, 0)
    lib = ibwd.library()
    base = [A, A + 0x100000, A + 0x200000, A + 0x400000, A + 0x500000, A + 0x600000, A + 0x700000,
            A + 0x800000]
    assert lib.indexer_bwd_dense(*base, 1, 16, 16, 4, 32, 0, 1.0, 1.0, SR, A + 0x1000000, 1 << 30,
                                 None) == ibwd.IBWD_ERR_INVALID_ARGUMENT
    # the binding names the routes
    with pytest.raises(ValueError):
        ibwd._flags(False, False, False, "sideways")
    assert ibwd._flags(False, False, False, "slot_rows") == SR
    assert ibwd._flags(True, False, True, "key_ranges") == KR | ibwd.IBWD_FLAG_DETERMINISTIC | ibwd.IBWD_FLAG_BF16_OUT


# fake, 256-byte aligned "device" addresses: every case below must be rejected
# by host-side validation, so nothing is dereferenced
A = 0x10000000


def sparse_args(**kw):
    a = dict(q=A, k=A + 0x100000, w=A + 0x200000, ids=A + 0x300000, I=A + 0x400000, p=A + 0x500000,
             dq=A + 0x600000, dw=A + 0x700000, dk=A + 0x800000, B=1, S_q=64, S_k=128, H=4, D=32,
             topk=16, sm=1.0, gl=1.0, flags=0, ws=A + 0x1000000, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return a


def call_sparse(a):
    lib = ibwd.library()
    return lib.indexer_bwd_sparse(a["q"], a["k"], a["w"], a["ids"], a["I"], a["p"], a["dq"], a["dw"],
                                  a["dk"], a["B"], a["S_q"], a["S_k"], a["H"], a["D"], a["topk"],
                                  a["sm"], a["gl"], a["flags"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("bad", [
    dict(q=None), dict(k=None), dict(w=None), dict(ids=None), dict(I=None), dict(p=None),
    dict(dq=None), dict(dw=None), dict(dk=None),
    dict(B=0), dict(S_q=0), dict(S_k=-1), dict(H=0), dict(H=65), dict(D=48), dict(D=256),
    dict(topk=0), dict(topk=129), dict(topk=129, flags=2, ws=None, ws_bytes=0), dict(flags=3), dict(flags=7), dict(flags=10), dict(flags=64), dict(flags=48),
    dict(flags=2 | 16, ws=None, ws_bytes=0), dict(flags=2 | 32, ws=None, ws_bytes=0), dict(q=A + 8), dict(dk=A + 0x800004),
    dict(w=A + 0x200002), dict(ws=None, ws_bytes=0), dict(ws=A + 0x900000, ws_bytes=16),
    dict(ws=A + 0x900010, ws_bytes=1 << 30), dict(flags=1, ws=None, ws_bytes=1 << 30),
    dict(B=1 << 20, S_q=1 << 20, H=64, D=128), dict(S_k=1024 * 256 + 1, D=128, ws_bytes=1 << 40),
])
def test_sparse_rejects_invalid_arguments(bad):
    assert call_sparse(sparse_args(**bad)) == ibwd.IBWD_ERR_INVALID_ARGUMENT


def test_dense_rejects_invalid_arguments():
    lib = ibwd.library()
    base = [A, A + 0x100000, A + 0x200000, A + 0x400000, A + 0x500000, A + 0x600000, A + 0x700000,
            A + 0x800000]
    assert lib.indexer_bwd_dense(*base[:3], None, *base[4:], 1, 16, 16, 4, 32, 0, 1.0, 1.0, 2, None,
                                 0, None) == ibwd.IBWD_ERR_INVALID_ARGUMENT
    # default route without workspace
    assert lib.indexer_bwd_dense(*base, 1, 16, 16, 4, 32, 0, 1.0, 1.0, 0, None, 0,
                                 None) == ibwd.IBWD_ERR_INVALID_ARGUMENT
    assert lib.indexer_bwd_dense(*base, 1, 16, 16, 4, 40, 0, 1.0, 1.0, 0, None, 0,
                                 None) == ibwd.IBWD_ERR_INVALID_ARGUMENT
    assert lib.indexer_bwd_dense(*base, 1, 16, 0, 4, 32, 0, 1.0, 1.0, 0, None, 0,
                                 None) == ibwd.IBWD_ERR_INVALID_ARGUMENT
    # the dense call has no ids, so the global-id flag is an error there
    for flags in (ibwd.IBWD_FLAG_GLOBAL_IDS, ibwd.IBWD_FLAG_GLOBAL_IDS | ibwd.IBWD_FLAG_ATOMIC_DK,
                  ibwd.IBWD_FLAG_BF16_OUT | ibwd.IBWD_FLAG_ATOMIC_DK):
        assert lib.indexer_bwd_dense(*base, 1, 16, 16, 4, 32, 0, 1.0, 1.0, flags, A + 0x1000000,
                                     1 << 30, None) == ibwd.IBWD_ERR_INVALID_ARGUMENT


def test_valid_arguments_without_gpu_fail_cleanly():
    """With valid arguments the call reaches the device check; on a machine
    without a gfx950 GPU it must report an error, not crash or launch."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: covered by the GPU tests")
    G = ibwd.IBWD_FLAG_GLOBAL_IDS
    for a in (sparse_args(), sparse_args(flags=ibwd.IBWD_FLAG_ATOMIC_DK, ws=None, ws_bytes=0),
              sparse_args(flags=G), sparse_args(flags=G | ibwd.IBWD_FLAG_DETERMINISTIC),
              sparse_args(flags=G | ibwd.IBWD_FLAG_ATOMIC_DK, ws=None, ws_bytes=0),
              sparse_args(flags=ibwd.IBWD_FLAG_BF16_OUT),
              sparse_args(flags=G | ibwd.IBWD_FLAG_BF16_OUT | ibwd.IBWD_FLAG_DETERMINISTIC),
              sparse_args(flags=ibwd.IBWD_FLAG_DK_SLOT_ROWS), sparse_args(flags=ibwd.IBWD_FLAG_DK_KEY_RANGES)):
        assert call_sparse(a) in (ibwd.IBWD_ERR_HIP, ibwd.IBWD_ERR_UNSUPPORTED_DEVICE)


def test_stage_hook_set_and_remove_without_gpu():
    """The profiling hook installs and uninstalls; a call rejected before launch
    (invalid arguments) reports no kernel to it."""
    seen = []
    ibwd.set_stage_hook(lambda stage, name: seen.append((stage, name)))
    try:
        lib = ibwd.library()
        st = lib.indexer_bwd_sparse(*([None] * 9), 1, 4, 16, 4, 32, 4, 1.0, 1.0, 0, None, 0, None)
        assert st == ibwd.IBWD_ERR_INVALID_ARGUMENT
    finally:
        ibwd.set_stage_hook(None)
    assert seen == []
    assert ibwd.library().indexer_bwd_set_stage_hook(ibwd._HOOK_T(), None) == ibwd.IBWD_OK


def test_forward_and_topk_reject_invalid_arguments():
    lib = ibwd.library()
    q, k, w, sc = A, A + 0x100000, A + 0x200000, A + 0x300000

    def fwd(**kw):
        a = dict(q=q, k=k, w=w, sc=sc, B=1, S_q=16, S_k=64, H=4, D=32, causal=0, off=0)
        a.update(kw)
        return lib.indexer_fwd_scores(a["q"], a["k"], a["w"], a["sc"], a["B"], a["S_q"], a["S_k"],
                                      a["H"], a["D"], a["causal"], a["off"], None)

    for bad in (dict(q=None), dict(k=None), dict(w=None), dict(sc=None), dict(B=0), dict(S_k=0),
                dict(H=65), dict(D=48), dict(q=A + 8), dict(sc=A + 0x300002), dict(off=1 << 41),
                dict(S_q=1 << 16, S_k=1 << 16)):
        assert fwd(**bad) == ibwd.IBWD_ERR_INVALID_ARGUMENT, bad

    def topk(**kw):
        a = dict(sc=sc, ids=A + 0x400000, vals=A + 0x500000, rows=8, S_k=64, topk=16)
        a.update(kw)
        return lib.indexer_topk(a["sc"], a["ids"], a["vals"], a["rows"], a["S_k"], a["topk"], None)

    for bad in (dict(sc=None), dict(ids=None), dict(rows=0), dict(S_k=0), dict(topk=0),
                dict(topk=65), dict(ids=A + 0x400002), dict(vals=A + 0x500001),
                dict(rows=1 << 20, S_k=1 << 12)):
        assert topk(**bad) == ibwd.IBWD_ERR_INVALID_ARGUMENT, bad


def test_forward_and_topk_without_gpu_fail_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: covered by the GPU tests")
    lib = ibwd.library()
    assert lib.indexer_fwd_scores(A, A + 0x100000, A + 0x200000, A + 0x300000, 1, 16, 64, 4, 32, 1,
                                  0, None) in (ibwd.IBWD_ERR_HIP, ibwd.IBWD_ERR_UNSUPPORTED_DEVICE)
    assert lib.indexer_topk(A, A + 0x400000, None, 8, 64, 16, None) in (
        ibwd.IBWD_ERR_HIP, ibwd.IBWD_ERR_UNSUPPORTED_DEVICE)


def test_binding_allocates_the_workspace_on_the_launch_stream(monkeypatch):
    """A workspace the binding allocates belongs to the stream the kernels run
    on (it is released when the call returns; the caching allocator may then
    reuse it only in that stream's order)."""
    torch = pytest.importorskip("torch")
    import contextlib

    entered = []

    @contextlib.contextmanager
    def fake_stream(s):
        entered.append(s)
        try:
            yield
        finally:
            entered.pop()

    made = []
    real_empty = torch.empty

    def fake_empty(*a, **kw):
        made.append(entered[-1] if entered else None)
        kw["device"] = "cpu"
        return real_empty(*a, **kw)

    monkeypatch.setattr(torch.cuda, "stream", fake_stream)
    monkeypatch.setattr(torch, "empty", fake_empty)
    side = object()
    ws, nbytes = ibwd._workspace(False, 1, 64, 128, 4, 32, 16, 0, None, "cpu", side)
    assert made == [side]
    assert nbytes == ibwd.indexer_bwd_workspace_bytes(False, 1, 64, 128, 4, 32, 16, 0) > 0
    # a caller's workspace is used as given; the atomic route needs none
    assert ibwd._workspace(False, 1, 64, 128, 4, 32, 16, 0, ws, "cpu", side)[0] is ws
    assert ibwd._workspace(False, 1, 64, 128, 4, 32, 16, ibwd.IBWD_FLAG_ATOMIC_DK, None, "cpu",
                           side) == (None, 0)
    assert made == [side]
