"""GPU parity of the fp8 grouped expert GEMM (moe_expert_gemm_fp8) against
the oracle's blocked fp64 definition, through the C ABI.

The oracle's routing is handed to the GPU (moe_plan); the GPU dispatches in
fp8 and the GEMM reads that buffer; the oracle recomputes the dispatched
rows itself.  Outputs agree within the rounding bound of the kernel's
arithmetic; padding rows inside a segment are zero; rows past the last
segment are never written.
"""
import numpy as np
import pytest
import torch

from combine_router_gate_amd import inputs as I
from combine_router_gate_amd import moe
from oracle import moe_oracle as O
from _gpu_common import check_bf16_close, note, to_dev, to_host, torch_dtype

pytestmark = pytest.mark.gpu

C = I.CONFIGS
U = 2.0 ** -24
SENTINEL = 7.0

CASES = {
    # name: (config, N, y dtype)
    "e8_pad16_n256": (C["dsv3_prefill"].with_shape(T=200, H=512, E=8, k=2,
                                                   pad=16), 256, "bf16"),
    "e16_pad128_n384": (C["dsv3_prefill"].with_shape(T=300, H=768, E=16, k=4,
                                                     pad=128), 384, "bf16"),
    "e40_k5_f32": (C["dsv3_prefill"].with_shape(T=150, H=256, E=40, k=5,
                                                pad=8), 128, "f32"),
    "e64_k8_k1024": (C["dsv3_decode"].with_shape(T=128, H=1024, E=64,
                                                 payload="fp8"), 512, "bf16"),
    # segments of ~300 rows: several row tiles per expert, a half-empty last
    "e4_long_segments": (C["dsv3_prefill"].with_shape(T=600, H=256, E=4, k=2,
                                                      pad=128), 384, "f32"),
    # the most experts (tile map over 1024 segments, many empty)
    "e1024": (C["moonep_skew"].with_shape(T=300, H=256, E=1024, k=4, pad=8,
                                          zipf_bias=False), 128, "bf16"),
}


# The gfx950 fp8 matrix instruction sums a block's 128 products with about
# 13 bits of relative precision: over 10^6 random tiles its error reached
# 2^-12.2 of sum|p| (2^-10.8 of the largest product).  Bound: 2^-9 of the
# block's sum|p| (4x margin), plus fp32 roundings for the scale product, the
# scaled add and the block accumulation.
MFMA_BLOCK_REL = 2.0 ** -9


def _bound(rows, scales, w, sw, e, K):
    mag = O.expert_gemm_fp8(rows & 0x7F, scales, w[e:e + 1] & 0x7F,
                            sw[e:e + 1], 0)
    return (MFMA_BLOCK_REL + (K // 128 + 4) * U) * mag


def _check(got, want, bound, ydt, what):
    if ydt == "f32":
        err = np.abs(np.asarray(got, np.float64) - want)
        assert (err <= bound + 1e-30).all(), (what, err.max())
    else:
        err = check_bf16_close(got, want, tol=bound + 1e-30, what=what)
    # and the fp8 path's absolute bar on these O(1) outputs
    g = np.asarray(got, np.float64) if ydt == "f32" else O.bf16_value(got)
    _, ex = np.frexp(want)
    half_ulp = 0.0 if ydt == "f32" else np.ldexp(1.0, np.maximum(ex, -125) - 9)
    assert (np.abs(g - want) <= 1e-2 + half_ulp).all(), what


def _run(cfg, seed, N, ydt, experts=None):
    wl = I.make_workload(cfg, seed)
    o = O.route(wl.x.values, wl.w_gate.values, wl.bias, cfg.k, cfg.pad)
    p = moe.plan(to_dev(o["topk_idx"]), cfg.E, cfg.pad)
    d = moe.dispatch(to_dev(wl.x), p, payload="fp8")
    w, sw = I.expert_weights_fp8(seed, cfg.E, N, cfg.H, experts=experts)
    cap = d["rows"].shape[0]
    y = torch.full((cap, N), SENTINEL, dtype=torch_dtype(ydt), device="cuda")
    ws = torch.empty(moe.moe_expert_gemm_workspace_bytes(cap, cfg.E),
                     dtype=torch.uint8, device="cuda")
    moe.moe_expert_gemm_fp8(d["rows"], d["row_scales"], d["row_src"],
                            p["offsets"], to_dev(w), to_dev(sw), y, ws)
    torch.cuda.synchronize()
    o_tok, o_src = O.assign_slots(o["topk_idx"], o["offsets"], cfg.E, cap)
    return wl, o, o_src, w, sw, y


def _gemm_case(name, cfg, N, ydt, seed=31):
    """Every routed row of every expert against the blocked fp64 oracle;
    padding rows zero, rows past the segments untouched."""
    note(f"expert gemm {name} T={cfg.T} K={cfg.H} N={N} E={cfg.E} "
         f"pad={cfg.pad} y={ydt}")
    wl, o, o_src, w, sw, y = _run(cfg, seed, N, ydt)
    rows_o, sc_o = O.dispatch_rows(wl.x.values, o_src, "fp8")
    got = to_host(y)
    for e in range(cfg.E):
        lo, c = int(o["offsets"][e]), int(o["counts"][e])
        if c == 0:
            continue
        seg = np.arange(lo, lo + c)
        want = O.expert_gemm_fp8(rows_o[seg], sc_o[seg], w, sw, e)
        bnd = _bound(rows_o[seg], sc_o[seg], w, sw, e, cfg.H)
        _check(got[seg], want, bnd, ydt, f"expert {e}")
    R = int(o["offsets"][-1])
    pad_rows = np.nonzero(o_src[:R] < 0)[0]
    assert not got[pad_rows].any(), "padding rows must be zero"
    tail = got[R:]
    if ydt == "f32":
        assert (tail == SENTINEL).all()
    else:
        assert (O.bf16_value(tail) == SENTINEL).all()


@pytest.mark.parametrize("name", list(CASES))
def test_expert_gemm_small(name):
    cfg, N, ydt = CASES[name]
    _gemm_case(name, cfg, N, ydt)


def test_expert_gemm_empty_experts():
    """Experts with no tokens own no tile; every token on expert 0."""
    cfg = C["dsv3_prefill"].with_shape(T=130, H=256, E=8, k=1, pad=128)
    note("expert gemm, all tokens on one expert")
    wl = I.make_workload(cfg, 3)
    idx = np.zeros((cfg.T, 1), np.int32)
    p = moe.plan(to_dev(idx), cfg.E, cfg.pad)
    d = moe.dispatch(to_dev(wl.x), p, payload="fp8")
    w, sw = I.expert_weights_fp8(3, cfg.E, 128, cfg.H)
    y = moe.expert_gemm_fp8(d, p, to_dev(w), to_dev(sw),
                            y_dtype=torch.float32)
    torch.cuda.synchronize()
    rows_o, sc_o = O.dispatch_rows(wl.x.values, np.arange(cfg.T), "fp8")
    want = O.expert_gemm_fp8(rows_o, sc_o, w, sw, 0)
    bnd = _bound(rows_o, sc_o, w, sw, 0, cfg.H)
    _check(to_host(y)[:cfg.T], want, bnd, "f32", "expert 0")
    assert not to_host(y)[cfg.T:256].any()


def test_expert_gemm_prefill_full_size_sampled():
    """DeepSeek-V3 prefill shape (T=16384, K=N=7168, E=256, fp8 dispatch):
    three experts carry random weights, the others zero; sampled rows of the
    three are checked against the oracle, sampled rows elsewhere are 0."""
    cfg = C["dsv3_prefill"]
    pick = [3, 128, 250]
    note(f"expert gemm dsv3_prefill full size, experts {pick}")
    wl, o, o_src, w, sw, y = _run(cfg, 0, cfg.H, "bf16", experts=pick)
    rng = np.random.default_rng(5)
    for e in pick:
        lo, c = int(o["offsets"][e]), int(o["counts"][e])
        seg = np.unique(np.concatenate([[lo, lo + c - 1],
                                        rng.integers(lo, lo + c, 14)]))
        rows_o = np.zeros((len(seg), cfg.H), np.uint8)
        sc_o = np.zeros((len(seg), cfg.H // 128), np.float32)
        for i, r in enumerate(seg):
            rows_o[i], sc_o[i] = O.dispatch_row(wl.x.values[o_src[r]], "fp8")
        want = O.expert_gemm_fp8(rows_o, sc_o, w, sw, e)
        bnd = _bound(rows_o, sc_o, w, sw, e, cfg.H)
        got = to_host(y[torch.from_numpy(seg).cuda()])
        _check(got, want, bnd, "bf16", f"expert {e}")
    others = [e for e in range(cfg.E) if e not in pick][::37]
    rs = np.array([int(o["offsets"][e]) for e in others])
    assert not to_host(y[torch.from_numpy(rs).cuda()]).any()


def test_expert_gemm_deterministic():
    """The grouped GEMM gives the same bits on every call."""
    cfg, N, ydt = next(iter(CASES.values()))
    note(f"expert gemm determinism T={cfg.T} K={cfg.H} N={N} E={cfg.E}")
    wl = I.make_workload(cfg, 37)
    o = O.route(wl.x.values, wl.w_gate.values, wl.bias, cfg.k, cfg.pad)
    p = moe.plan(to_dev(o["topk_idx"]), cfg.E, cfg.pad)
    d = moe.dispatch(to_dev(wl.x), p, payload="fp8")
    w, sw = I.expert_weights_fp8(37, cfg.E, N, cfg.H)
    w, sw = to_dev(w), to_dev(sw)
    cap = d["rows"].shape[0]
    ws = torch.empty(moe.moe_expert_gemm_workspace_bytes(cap, cfg.E),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        y = torch.zeros((cap, N), dtype=torch_dtype(ydt), device="cuda")
        moe.moe_expert_gemm_fp8(d["rows"], d["row_scales"], d["row_src"],
                                p["offsets"], w, sw, y, ws)
        torch.cuda.synchronize()
        outs.append(y.view(torch.int16 if ydt == "bf16" else torch.int32))
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
