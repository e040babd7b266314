"""C-ABI library: loads, exports every declared symbol, and rejects invalid
arguments on the host before anything is enqueued.  CPU only.

Pointer arguments here are fake addresses that are never dereferenced: each
call violates exactly one precondition, so validation returns before any
kernel launch.  The tests skip on a machine with a GPU, where a validation
bug would launch a kernel on those addresses; GPU-side error handling is
covered with real tensors in the GPU tests.
"""
import ctypes

import pytest

from combine_router_gate_amd import moe
from combine_router_gate_amd import build as B
from oracle import moe_oracle as O

OK, NULL, SHAPE, DTYPE, ALIGN, CAP, WS, ALIAS = 0, -1, -2, -3, -4, -5, -6, -7
SCRATCH = -9


@pytest.fixture(scope="module")
def L():
    import os
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("library not built")
    return moe.lib()


@pytest.fixture(scope="module")
def no_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation tests run only without a GPU")


def test_exports_every_header_symbol(L):
    names = moe.header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    dl = ctypes.CDLL(B.LIB_PATH)
    for n in ["moe_route", "moe_plan", "moe_dispatch", "moe_combine_residual"]:
        assert getattr(dl, n) is not None


def test_status_strings(L):
    for s in [OK, NULL, SHAPE, DTYPE, ALIGN, CAP, WS, ALIAS, -8, SCRATCH]:
        txt = moe.moe_status_string(s)
        assert txt and "unknown" not in txt
    assert "unknown" in moe.moe_status_string(-99)


@pytest.mark.parametrize("T,E,k,pad", [(64, 8, 2, 1), (4096, 8, 2, 128),
                                       (128, 256, 8, 128), (16384, 256, 8, 128),
                                       (8192, 384, 8, 128), (0, 8, 2, 4)])
def test_capacity_formula(L, T, E, k, pad):
    assert moe.moe_rows_capacity(T, E, k, pad) == O.rows_capacity(T, E, k, pad)


def test_capacity_invalid(L):
    assert moe.moe_rows_capacity(10, 4, 5, 1) == 0      # k > E
    assert moe.moe_rows_capacity(10, 0, 1, 1) == 0
    assert moe.moe_rows_capacity(10, 1025, 2, 1) == 0
    assert moe.moe_rows_capacity(10, 8, 17, 1) == 0
    assert moe.moe_rows_capacity(10, 8, 2, 0) == 0
    assert moe.moe_rows_capacity(2 ** 30, 8, 8, 1) == 0  # rows overflow int32


def test_workspace_bytes(L):
    assert moe.moe_workspace_bytes(0, 8, 2) == 0
    w = moe.moe_workspace_bytes(16384, 256, 8)
    assert w >= 4 * (256 * 256 + 16384 * 8)
    assert moe.moe_workspace_bytes(65, 8, 2) >= 4 * (2 * 8 + 65 * 2)
    # room for the split gate's partial logits: up to 4 hidden ranges of
    # fp32 [T, 64 * ceil(E / 64)] through 65536 tokens, none beyond
    for T, E in ((20000, 256), (65536, 512), (4096, 384)):
        tiles = 4 * ((T + 63) // 64) * E + 4 * T * 8
        assert moe.moe_workspace_bytes(T, E, 8) >= tiles + 4 * 4 * T * 64 * (
            (E + 63) // 64)
    T = 65537
    assert moe.moe_workspace_bytes(T, 256, 8) < 2 * 4 * T * 256


# fake, 256-aligned, far-apart device addresses (never dereferenced)
A = [0x10000000 * (i + 1) for i in range(16)]


def _route(L, **kw):
    a = dict(x=A[0], xdt=1, T=100, H=256, w=A[1], E=16, bias=None, k=2, pad=4,
             idx=A[2], tw=A[3], counts=A[4], offsets=A[5], dbg=None, ws=A[6],
             wsb=1 << 26, stream=None)
    a.update(kw)
    return L.moe_route(a["x"], a["xdt"], a["T"], a["H"], a["w"], a["E"],
                       a["bias"], a["k"], a["pad"], a["idx"], a["tw"],
                       a["counts"], a["offsets"], a["dbg"], a["ws"], a["wsb"],
                       a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(idx=None), NULL),
    (dict(counts=None), NULL), (dict(ws=None), NULL),
    (dict(k=17), SHAPE), (dict(k=0), SHAPE), (dict(E=0), SHAPE),
    (dict(E=1025), SHAPE), (dict(k=20, E=16), SHAPE), (dict(H=12), SHAPE),
    # above 512 experts the gate takes bf16 x and at most 65536 tokens
    (dict(E=600, xdt=0), DTYPE), (dict(E=600, T=65537), SHAPE),
    (dict(H=0), SHAPE), (dict(T=-1), SHAPE), (dict(pad=0), SHAPE),
    (dict(xdt=2), DTYPE), (dict(xdt=7), DTYPE),
    (dict(x=A[0] + 8), ALIGN), (dict(w=A[1] + 4), ALIGN),
    (dict(wsb=100), WS),
    (dict(tw=A[0]), ALIAS), (dict(idx=A[1] + 64), ALIAS),
    (dict(dbg=A[4]), ALIAS), (dict(ws=A[5] - 256), ALIAS),
])
def test_route_validation(L, no_gpu, kw, want):
    assert _route(L, **kw) == want


def _dispatch(L, **kw):
    a = dict(x=A[0], xdt=1, T=100, H=256, idx=A[1], k=2, E=16, pad=4,
             counts=A[2], offsets=A[3], ws=A[4], wsb=1 << 26, pdt=1,
             rows=A[5], cap=O.rows_capacity(100, 16, 2, 4), scales=None,
             row_src=A[6], tok_row=A[7], stream=None)
    a.update(kw)
    return L.moe_dispatch(a["x"], a["xdt"], a["T"], a["H"], a["idx"], a["k"],
                          a["E"], a["pad"], a["counts"], a["offsets"], a["ws"],
                          a["wsb"], a["pdt"], a["rows"], a["cap"], a["scales"],
                          a["row_src"], a["tok_row"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(rows=None), NULL), (dict(row_src=None), NULL),
    (dict(pdt=2), NULL),                       # fp8 without scales
    (dict(scales=A[8]), DTYPE),                # scales without fp8
    (dict(pdt=0), DTYPE), (dict(xdt=2, pdt=2, scales=A[8]), DTYPE),
    (dict(pdt=2, scales=A[8], H=200), SHAPE),  # fp8 needs H % 128 == 0
    (dict(cap=O.rows_capacity(100, 16, 2, 4) - 1), CAP),
    (dict(wsb=10), WS), (dict(rows=A[5] + 4), ALIGN),
    (dict(rows=A[0]), ALIAS), (dict(tok_row=A[1]), ALIAS),
    (dict(row_src=A[4] + 128), ALIAS), (dict(k=0), SHAPE),
])
def test_dispatch_validation(L, no_gpu, kw, want):
    assert _dispatch(L, **kw) == want


def _route_dispatch(L, fn="moe_route_dispatch", **kw):
    a = dict(x=A[0], xdt=1, T=100, H=256, w=A[1], E=16, bias=None, k=2, pad=4,
             idx=A[2], tw=A[3], counts=A[4], offsets=A[5], dbg=None, ws=A[6],
             wsb=1 << 26, pdt=1, rows=A[7],
             cap=O.rows_capacity(100, 16, 2, 4), scales=None, row_src=A[8],
             tok_row=A[9], stream=None)
    a.update(kw)
    return getattr(L, fn)(
        a["x"], a["xdt"], a["T"], a["H"], a["w"], a["E"], a["bias"], a["k"],
        a["pad"], a["idx"], a["tw"], a["counts"], a["offsets"], a["dbg"],
        a["ws"], a["wsb"], a["pdt"], a["rows"], a["cap"], a["scales"],
        a["row_src"], a["tok_row"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(rows=None), NULL),
    (dict(ws=None), NULL), (dict(row_src=None), NULL), (dict(pdt=2), NULL),
    (dict(scales=A[10]), DTYPE), (dict(xdt=2), DTYPE), (dict(pdt=0), DTYPE),
    (dict(pdt=2, scales=A[10], H=200), SHAPE), (dict(k=17), SHAPE),
    (dict(E=1025), SHAPE), (dict(H=12), SHAPE),
    (dict(E=600, xdt=0, pdt=0), DTYPE),
    (dict(cap=O.rows_capacity(100, 16, 2, 4) - 1), CAP), (dict(wsb=10), WS),
    (dict(rows=A[7] + 4), ALIGN), (dict(ws=A[6] + 8), ALIGN),
    (dict(rows=A[0]), ALIAS), (dict(rows=A[6]), ALIAS),
    (dict(tok_row=A[2]), ALIAS), (dict(row_src=A[1]), ALIAS),
])
def test_route_dispatch_validation(L, no_gpu, kw, want):
    assert _route_dispatch(L, **kw) == want


ONE = "moe_route_dispatch_one_launch"


@pytest.mark.parametrize("kw,want", [
    # the checks of moe_route_dispatch come first
    (dict(x=None), NULL), (dict(rows=None), NULL), (dict(k=17), SHAPE),
    (dict(cap=O.rows_capacity(100, 16, 2, 4) - 1), CAP), (dict(wsb=10), WS),
    (dict(rows=A[0]), ALIAS),
    # then bf16 x, at most 256 tokens and 512 experts
    (dict(xdt=0, pdt=0), DTYPE),
    (dict(T=257, cap=O.rows_capacity(257, 16, 2, 4)), SHAPE),
    (dict(E=600, cap=O.rows_capacity(100, 600, 2, 4)), SHAPE),
])
def test_route_dispatch_one_launch_validation(L, no_gpu, kw, want):
    assert _route_dispatch(L, fn=ONE, **kw) == want


def _dispatch_noalloc(L, **kw):
    a = dict(x=A[0], xdt=1, T=100, H=256, idx=A[1], k=2, E=16, pad=4,
             counts=A[2], offsets=A[3], pdt=1, rows=A[5],
             cap=O.rows_capacity(100, 16, 2, 4), scales=None, row_src=A[6],
             tok_row=A[7], stream=None)
    a.update(kw)
    return L.moe_dispatch_noalloc(
        a["x"], a["xdt"], a["T"], a["H"], a["idx"], a["k"], a["E"], a["pad"],
        a["counts"], a["offsets"], a["pdt"], a["rows"], a["cap"], a["scales"],
        a["row_src"], a["tok_row"], a["stream"])


def _noalloc_cap(T, E, k, pad):
    return O.rows_capacity(T, E, k, pad)


@pytest.mark.parametrize("kw,want", [
    (dict(x=None), NULL), (dict(rows=None), NULL), (dict(row_src=None), NULL),
    (dict(pdt=2), NULL), (dict(scales=A[8]), DTYPE), (dict(pdt=0), DTYPE),
    (dict(pdt=2, scales=A[8], H=200), SHAPE),
    (dict(cap=O.rows_capacity(100, 16, 2, 4) - 1), CAP),
    (dict(rows=A[5] + 4), ALIGN), (dict(rows=A[0]), ALIAS),
    (dict(tok_row=A[1]), ALIAS), (dict(k=0), SHAPE), (dict(E=1025), SHAPE),
    # more slots and tile counts than the 8 MiB static scratch holds
    (dict(T=300000, H=8, k=8, E=16, cap=_noalloc_cap(300000, 16, 8, 4)),
     SCRATCH),
    (dict(T=90000, H=8, k=16, E=512, cap=_noalloc_cap(90000, 512, 16, 4)),
     SCRATCH),
])
def test_dispatch_noalloc_validation(L, no_gpu, kw, want):
    assert _dispatch_noalloc(L, **kw) == want


def test_noalloc_scratch_limit(L):
    limit = 8 << 20
    # every E and k the library accepts fits at 65536 tokens
    assert moe.moe_noalloc_scratch_bytes(65536, 512, 16) <= limit
    assert moe.moe_noalloc_scratch_bytes(16384, 256, 8) <= limit
    assert moe.moe_noalloc_scratch_bytes(300000, 16, 8) > limit
    assert moe.moe_noalloc_scratch_bytes(4, 0, 1) == 0
    # at least the tile bases and ranks the workspace would hold
    for T, E, k in ((100, 16, 2), (16384, 256, 8), (65536, 512, 16)):
        tiles = 4 * ((T + 63) // 64) * E + 4 * T * k
        assert moe.moe_noalloc_scratch_bytes(T, E, k) >= tiles


def _combine(L, **kw):
    a = dict(y=A[0], ydt=1, H=256, y_rows=1000, tok_row=A[1], tw=A[2], T=100,
             k=2, shared=A[3], res_in=A[4], res_out=A[5], rnr=A[6], out=None,
             odt=1, stream=None)
    a.update(kw)
    return L.moe_combine_residual(a["y"], a["ydt"], a["H"], a["y_rows"],
                                  a["tok_row"], a["tw"], a["T"], a["k"],
                                  a["shared"], a["res_in"], a["res_out"],
                                  a["rnr"], a["out"], a["odt"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(y=None), NULL), (dict(res_out=None), NULL),
    (dict(rnr=None, res_out=A[4] + 64), ALIAS),             # split form, partial overlap
    (dict(out=A[7]), ALIAS),                                  # out with residual
    (dict(res_in=None, res_out=None, rnr=None), NULL),        # no out at all
    (dict(res_in=None, out=A[7]), ALIAS),                     # stray residual_out
    (dict(res_in=None, res_out=None, rnr=None, out=A[7], odt=2), DTYPE),
    (dict(ydt=2), DTYPE), (dict(H=100), SHAPE), (dict(k=17), SHAPE),
    (dict(y=A[0] + 4), ALIGN), (dict(res_out=A[5] + 2), ALIGN),
    (dict(rnr=A[4]), ALIAS), (dict(res_out=A[4] + 256), ALIAS),
    (dict(res_out=A[3]), ALIAS), (dict(rnr=A[0]), ALIAS),
])
def test_combine_validation(L, no_gpu, kw, want):
    assert _combine(L, **kw) == want


def test_plan_validation(L, no_gpu):
    cap_ok = dict(idx=A[0], T=10, k=2, E=8, pad=1, counts=A[1], offsets=A[2],
                  ws=A[3], wsb=1 << 26)

    def call(**kw):
        a = dict(cap_ok)
        a.update(kw)
        return L.moe_plan(a["idx"], a["T"], a["k"], a["E"], a["pad"],
                          a["counts"], a["offsets"], a["ws"], a["wsb"], None)
    assert call(idx=None) == NULL
    assert call(counts=None) == NULL
    assert call(k=9) == SHAPE
    assert call(wsb=1) == WS
    assert call(counts=A[0]) == ALIAS
    assert call(counts=A[1] + 2) == ALIGN


def test_farskip_aux_validation(L, no_gpu):
    def call(**kw):
        a = dict(shared=A[0], res_in=A[1], rnr=A[2], T=100, H=256)
        a.update(kw)
        return L.moe_farskip_aux(a["shared"], a["res_in"], a["rnr"], a["T"],
                                 a["H"], None)
    assert call(T=-1) == SHAPE
    assert call(H=12) == SHAPE
    assert call(res_in=None) == NULL
    assert call(rnr=None) == NULL
    assert call(rnr=A[2] + 8) == ALIGN
    assert call(rnr=A[1] + 256) == ALIAS
    assert call(rnr=A[0]) == ALIAS
    assert call(T=0, res_in=None, rnr=None) == OK       # empty: nothing to do


def test_combine_backward_validation(L, no_gpu):
    def call(**kw):
        a = dict(g=A[0], y=A[1], ydt=1, H=256, y_rows=1000, tok_row=A[2],
                 tw=A[3], T=100, k=2, gy=A[4], gw=A[5])
        a.update(kw)
        return L.moe_combine_backward(a["g"], a["y"], a["ydt"], a["H"],
                                      a["y_rows"], a["tok_row"], a["tw"],
                                      a["T"], a["k"], a["gy"], a["gw"], None)
    assert call(k=0) == SHAPE
    assert call(H=100) == SHAPE
    assert call(ydt=2) == DTYPE
    for name in ["g", "y", "tok_row", "tw", "gy", "gw"]:
        assert call(**{name: None}) == NULL, name
    assert call(gy=A[4] + 4) == ALIGN
    assert call(gw=A[5] + 2) == ALIGN
    assert call(gy=A[1]) == ALIAS
    assert call(gw=A[3]) == ALIAS
    assert call(gy=A[0] + 512) == ALIAS


def test_dispatch_backward_validation(L, no_gpu):
    def call(**kw):
        a = dict(gr=A[0], rdt=1, H=256, cap=1000, tok_row=A[1], T=100, k=2,
                 gx=A[2], xdt=0)
        a.update(kw)
        return L.moe_dispatch_backward(a["gr"], a["rdt"], a["H"], a["cap"],
                                       a["tok_row"], a["T"], a["k"], a["gx"],
                                       a["xdt"], None)
    assert call(k=17) == SHAPE
    assert call(H=4) == SHAPE
    assert call(rdt=2) == DTYPE
    assert call(xdt=2) == DTYPE
    assert call(gr=None) == NULL
    assert call(gx=None) == NULL
    assert call(gx=A[2] + 8) == ALIGN
    assert call(gx=A[0] + 256) == ALIAS
    assert call(gx=A[1]) == ALIAS


def test_expert_gemm_validation(L, no_gpu):
    cap = 1024
    wsb = moe.moe_expert_gemm_workspace_bytes(cap, 8)
    assert wsb >= 8 * (cap // 256 + 8)
    assert moe.moe_expert_gemm_workspace_bytes(cap, 0) == 0

    def call(**kw):
        a = dict(rows=A[0], rsc=A[1], K=512, cap=cap, src=A[2], offs=A[3],
                 E=8, w=A[4], wsc=A[5], N=256, y=A[6], ydt=1, ws=A[7],
                 wsb=wsb)
        a.update(kw)
        return L.moe_expert_gemm_fp8(a["rows"], a["rsc"], a["K"], a["cap"],
                                     a["src"], a["offs"], a["E"], a["w"],
                                     a["wsc"], a["N"], a["y"], a["ydt"],
                                     a["ws"], a["wsb"], None)
    assert call(K=100) == SHAPE
    assert call(K=8192 + 128) == SHAPE
    assert call(N=200) == SHAPE
    assert call(E=0) == SHAPE
    assert call(ydt=2) == DTYPE
    assert call(cap=0, rows=None) == OK
    for name in ["rows", "rsc", "offs", "w", "wsc", "y", "ws"]:
        assert call(**{name: None}) == NULL, name
    assert call(wsb=wsb - 1) == WS
    assert call(y=A[6] + 8) == ALIGN
    assert call(rsc=A[1] + 2) == ALIGN
    assert call(y=A[4]) == ALIAS
    assert call(ws=A[6] + 256) == ALIAS
    assert call(ws=A[3]) == ALIAS
