"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

* route: GPU logits within LOGIT_TOL of the fp64 oracle, top-k equal where
  the choice is unique (near ties audited), counts/offsets bit-exact.
* integer inputs: exact logits on both sides, so routing (tie-breaks
  included), slots, rows and the whole chain must match bit for bit.
* dispatch / fixture / combine: the oracle's routing is handed to the GPU
  (moe_plan) so both sides start from the same choice; counts, offsets,
  tok_row, row_src, rows and fp8 scales bit-exact, combine within tolerance.
Small shapes are checked element by element; the five workload shapes at
full size on sampled rows and tokens.
"""
import numpy as np
import pytest
import torch

from combine_router_gate_amd import inputs as I
from combine_router_gate_amd import moe
from oracle import moe_oracle as O
from _gpu_common import (LOGIT_TOL, check_bf16_close, check_f32_close,
                         check_plan_valid, check_topk_own_logits, note,
                         to_dev, to_host, topk_audit, torch_dtype)

pytestmark = pytest.mark.gpu

C = I.CONFIGS
SMALL = {
    "tiny": C["tiny"],
    "mixtral_s": C["mixtral"].with_shape(T=300, H=512),
    "decode": C["dsv3_decode"],
    "prefill_s": C["dsv3_prefill"].with_shape(T=333, H=1024),
    "moonep_s": C["moonep_skew"].with_shape(T=517),
    "f32_wide": C["tiny"].with_shape(T=130, H=256, E=100, k=4, pad=3),
    "fp8_routed_f32": C["mixtral"].with_shape(T=70, H=256, E=20, k=3, pad=5,
                                              payload="fp8"),
    "f32_to_fp8": C["tiny"].with_shape(T=50, H=128, E=64, k=6, pad=2,
                                       payload="fp8", y_dtype="bf16",
                                       expert="scale"),
    "e512_k16": C["moonep_skew"].with_shape(T=100, H=64, E=512, k=16, pad=8,
                                            zipf_bias=False),
    "h8": C["mixtral"].with_shape(T=65, H=8, E=24, k=2, pad=1),
    "e40_k5": C["dsv3_decode"].with_shape(T=191, H=384, E=40, k=5, pad=16),
    "bf16_e100_h320": C["mixtral"].with_shape(T=130, H=320, E=100, k=4, pad=7),
    "bf16_e64_h200": C["mixtral"].with_shape(T=77, H=200, E=64, k=3, pad=2),
    "split_t1500": C["dsv3_decode"].with_shape(T=1500, H=1024),
    "split_t3000_e128": C["dsv3_prefill"].with_shape(T=3000, H=512, E=128,
                                                     k=6, pad=32),
    # few tokens: one-kernel reduction + plan, 24 and 32 expert tiles
    "small_e384": C["moonep_skew"].with_shape(T=200),
    "small_e512": C["moonep_skew"].with_shape(T=300, H=512, E=512,
                                              zipf_bias=False),
    "small_t512": C["dsv3_decode"].with_shape(T=512, H=1024, k=6, pad=16),
    "small_t1": C["dsv3_decode"].with_shape(T=1, H=2048),
    # many tokens: the LDS-staged partial gate (2 and 1 expert tiles per
    # wave, ragged token tile, 128-wide hidden ranges; gate weights of 1 MiB
    # and more, below which the narrow one-pass gate runs) and its fallback
    # for H not a multiple of 128
    "lds_gate_t4100_e100": C["dsv3_prefill"].with_shape(T=4100, H=5248, E=100,
                                                        k=6, pad=32),
    "lds_gate_t4096_e64": C["mixtral"].with_shape(T=4096, H=8192, E=64, k=4,
                                                  pad=16),
    "gate_t4096_h1032": C["dsv3_decode"].with_shape(T=4096, H=1032, E=256),
    # 34 tiles of 128 tokens (the last ragged), S = 4: workgroups mapped so
    # each XCD serves one hidden range
    "lds_gate_t4300_xcd": C["dsv3_prefill"].with_shape(T=4300, H=2048),
    # few experts (E <= 32) and many bf16 tokens take the LDS-staged gate too
    "lds_gate_t4200_e24": C["mixtral"].with_shape(T=4200, H=512, E=24, k=3,
                                                  pad=16),
    # 512 < T < 4096: 64-token tiles with expert groups of 64 (128 above
    # 2048 tokens), 4 or 8 hidden ranges; the reduction's range chunks
    # (S = 8 in chunks of 4, and of 2 for 24 and 32 expert tiles) and its
    # 16-token workgroups
    "reduce_t2048_s8": C["dsv3_prefill"].with_shape(T=2048, H=1024),
    "reduce_t2048_e384_s8": C["moonep_skew"].with_shape(T=2048, H=1024),
    "reduce_t1024_e512_s4": C["moonep_skew"].with_shape(T=1024, H=512, E=512,
                                                        zipf_bias=False),
    "reduce_t700_e256": C["dsv3_decode"].with_shape(T=700, H=1024),
    "reduce_t700_e384_s8": C["moonep_skew"].with_shape(T=700, H=1024),
    "mid_t2500_e256": C["dsv3_prefill"].with_shape(T=2500, H=1024),
    "mid_t4095_e100": C["mixtral"].with_shape(T=4095, H=384, E=100, k=4,
                                              pad=16),
    # the most experts (512) with many tokens: split gate with 64-token
    # tiles, reduction in chunks of two ranges
    "e512_t4096": C["moonep_skew"].with_shape(T=4096, H=1024, E=512, k=8,
                                              zipf_bias=False),
    # narrow one-pass gate (weight under 1 MiB, 4096..32768 tokens): 1, 2
    # and 4 expert tiles per wave (3 is the MoonEP workload), padded
    # experts, ragged last 32-token workgroup, a single 64-wide k step
    "narrow_t4097_e100": C["dsv3_prefill"].with_shape(T=4097, H=512, E=100,
                                                      k=6, pad=32),
    "narrow_t6000_e200_h640": C["moonep_skew"].with_shape(T=6000, H=640,
                                                          E=200),
    "narrow_t5000_e512": C["moonep_skew"].with_shape(T=5000, H=256, E=512,
                                                     zipf_bias=False),
    "narrow_t4100_h64": C["dsv3_decode"].with_shape(T=4100, H=64, E=256),
    # more than 512 experts: partial logits in expert groups of 256, a
    # 64-lane top-k per token (12 and 16 logits per lane), the plan kernels;
    # one workgroup per token up to 512 tokens, else one wave per token; a
    # single hidden range at H = 64
    "e1024_t100_k16": C["moonep_skew"].with_shape(T=100, H=256, E=1024, k=16,
                                                  pad=8, zipf_bias=False),
    "e1024_t1000_bias": C["moonep_skew"].with_shape(T=1000, H=512, E=1024),
    "e600_t5000": C["moonep_skew"].with_shape(T=5000, H=384, E=600,
                                              zipf_bias=False),
    "e1024_t700_h64": C["moonep_skew"].with_shape(T=700, H=64, E=1024,
                                                  zipf_bias=False),
}
FULL = ["mixtral", "dsv3_decode", "dsv3_prefill", "moonep_skew", "tiny"]
# gate shapes above 8192 tokens (route only: the dispatch and combine of
# these sizes are the full workloads' paths): 128-token tiles with 3 hidden
# ranges, and more than 16384 tokens (split gate, fused-histogram reduction)
ROUTE_ONLY = {
    "lds_gate_t10000_s3": C["dsv3_prefill"].with_shape(T=10000, H=2048),
    "lds_gate_t20000": C["dsv3_prefill"].with_shape(T=20000, H=2048),
    # first shapes past each policy boundary: 513 tokens (64-token tiles
    # with expert groups), 8193 (128-token tiles), 16321 (64-token
    # reduction workgroups that build the tile histogram)
    "mid_t513": C["dsv3_decode"].with_shape(T=513, H=512),
    "lds_gate_t8193": C["dsv3_prefill"].with_shape(T=8193, H=2048),
    "fused_hist_t16321": C["moonep_skew"].with_shape(T=16321, H=1408),
    # the narrow gate near its upper token bound
    "narrow_t32768": C["moonep_skew"].with_shape(T=32768, H=256),
}


def _route_gpu(wl):
    cfg = wl.cfg
    x, w = to_dev(wl.x), to_dev(wl.w_gate)
    b = to_dev(wl.bias) if wl.bias is not None else None
    return moe.route(x, w, cfg.k, cfg.pad, bias=b, want_logits=True), x


def _route_case(name, cfg, seed, sample_rows=64):
    """Route on the GPU, compare with the oracle, then dispatch from the
    route's own workspace (the plan the benchmark runs) and check the rows
    it produced."""
    note(f"route {name} seed={seed} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}")
    wl = I.make_workload(cfg, seed)
    p, x = _route_gpu(wl)
    d = moe.dispatch(x, p, payload="fp8" if cfg.payload == "fp8" else "same")
    torch.cuda.synchronize()
    o = O.route(wl.x.values, wl.w_gate.values, wl.bias, cfg.k, cfg.pad)
    gl = to_host(p["logits"])
    dl = np.abs(gl.astype(np.float64) - o["logits"]).max()
    assert dl <= LOGIT_TOL, dl
    gi, gw = to_host(p["topk_idx"]), to_host(p["topk_w"])
    check_topk_own_logits(gi, gw, gl, cfg.k)
    near = topk_audit(gi, gw, o["logits"], gl, cfg.k)
    counts, offs = to_host(p["counts"]), to_host(p["offsets"])
    tok_row, row_src = to_host(d["tok_row"]), to_host(d["row_src"])
    same = bool((gi == o["topk_idx"]).all())
    if same:
        cap = O.rows_capacity(cfg.T, cfg.E, cfg.k, cfg.pad)
        o_tok, o_src = O.assign_slots(o["topk_idx"], o["offsets"], cfg.E, cap)
        assert np.array_equal(counts, o["counts"])
        assert np.array_equal(offs, o["offsets"])
        assert np.array_equal(tok_row, o_tok)
        assert np.array_equal(row_src, o_src)
    else:   # a near tie went the other way: the plan must still be exact
        # for the GPU's own choice
        check_plan_valid(gi, counts, offs, tok_row, row_src, cfg.E, cfg.pad)
    # sampled rows of the payload (row_src verified above)
    valid = np.nonzero(row_src >= 0)[0]
    rsel = np.random.default_rng(seed).choice(
        valid, min(sample_rows, len(valid)), replace=False)
    ridx = torch.from_numpy(rsel.astype(np.int64)).cuda()
    g_rows = to_host(d["rows"][ridx])
    g_sc = to_host(d["row_scales"][ridx]) if cfg.payload == "fp8" else None
    for i, r in enumerate(rsel):
        pay, sc = O.dispatch_row(wl.x.values[row_src[r]], cfg.payload)
        assert np.array_equal(g_rows[i], pay), f"row {r}"
        if g_sc is not None:
            assert np.array_equal(g_sc[i], sc), f"scales of row {r}"
    note(f"route {name}: max|dlogit|={dl:.2e} near-ties={near} "
         f"plan={'oracle' if same else 'own top-k'}")


@pytest.mark.parametrize("name", list(SMALL))
def test_route_small(name):
    _route_case(name, SMALL[name], 1)


@pytest.mark.parametrize("name", list(ROUTE_ONLY))
def test_route_large(name):
    _route_case(name, ROUTE_ONLY[name], 1)


@pytest.mark.parametrize("name", FULL)
def test_route_full(name):
    _route_case(name, C[name], 0)


# ------------------------------------------------------------------ integer

INT_CASES = {
    "int_e8": C["mixtral"].with_shape(T=257, H=256, E=8, k=2, pad=4),
    "int_e256": C["dsv3_decode"].with_shape(T=200, H=512, E=256, k=8),
    "int_f32_e20": C["tiny"].with_shape(T=99, H=64, E=20, k=3, pad=2),
    "int_e384_fp8": C["moonep_skew"].with_shape(T=130, H=256, payload="fp8",
                                               zipf_bias=False),
    # many tokens (LDS-staged partial gate)
    "int_t4096_e256": C["dsv3_decode"].with_shape(T=4096, H=256, E=256, k=8),
}
# The route's own plan on the paths that build the tile histogram inside the
# gate's top-k epilogue, compared through dispatch, fixture and combine on
# sampled rows and tokens: the DeepSeek-V3 prefill shape itself (LDS-staged
# split gate, 64-token reduction workgroups with the fused histogram, fp8
# payload, dual residual), the first size with fused-histogram reduction
# workgroups at 384 experts, more than 16384 tokens, and the one-pass gate
# (hidden dimension not split: H = 64 at few and many tokens, and more
# tokens than the partial-logit workspace holds).
INT_LARGE = {
    "int_dsv3_prefill": C["dsv3_prefill"],
    # split gate + fused-histogram reduction (weights of 1 MiB and more)
    "int_fused_t16321_e384": C["moonep_skew"].with_shape(T=16321, H=1408,
                                                        zipf_bias=False),
    "int_t20000": C["dsv3_prefill"].with_shape(T=20000, H=2048),
    "int_onepass_t300_e512_k16": C["moonep_skew"].with_shape(
        T=300, H=64, E=512, k=16, pad=8, zipf_bias=False),
    # narrow one-pass gate, then tile histogram and parallel scan
    "int_narrow_t5000_h64": C["dsv3_decode"].with_shape(T=5000, H=64),
    "int_narrow_moonep": C["moonep_skew"].with_shape(zipf_bias=False),
    "int_onepass_t70000": C["mixtral"].with_shape(T=70000, H=128, E=64, k=4,
                                                  pad=16),
}


def _integer_chain(cfg, name, full_check):
    note(f"integer chain {name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} "
         f"payload={cfg.payload}")
    wl = I.integer_workload(cfg, 3)
    p, x = _route_gpu(wl)
    torch.cuda.synchronize()
    o = O.route(wl.x.values, wl.w_gate.values, None, cfg.k, cfg.pad)
    gl = to_host(p["logits"])
    assert np.array_equal(gl.astype(np.float64), o["logits"])
    gi = to_host(p["topk_idx"])
    check_topk_own_logits(gi, to_host(p["topk_w"]), gl, cfg.k)
    assert np.array_equal(gi, o["topk_idx"])
    np.testing.assert_allclose(to_host(p["topk_w"]), o["topk_w"], rtol=0,
                               atol=2e-6)
    assert np.array_equal(to_host(p["counts"]), o["counts"])
    assert np.array_equal(to_host(p["offsets"]), o["offsets"])
    _dispatch_combine_compare(wl, o, p, x, full_check=full_check)


@pytest.mark.parametrize("name", list(INT_CASES))
def test_integer_inputs_bit_exact_chain(name):
    """Integer x and W in {-2..2}: logits are exact integers on both sides,
    ties are frequent, and the chain from the GPU's own routing must equal
    the oracle's exactly (combine within tolerance)."""
    _integer_chain(INT_CASES[name], name, full_check=True)


@pytest.mark.parametrize("name", list(INT_LARGE))
def test_integer_route_plan_chain_large(name):
    """As above at sizes up to the full DeepSeek-V3 prefill shape: the slot
    plan moe_route writes (tile bases and ranks from its own epilogue)
    drives moe_dispatch, and tok_row / row_src must equal the oracle's in
    full; rows, scales, expert outputs and the combine on samples."""
    _integer_chain(INT_LARGE[name], name, full_check=False)


# ------------------------------------------------------------------ dispatch

def _oracle_rows(wl, row_src, rows_idx):
    """Oracle payload (and scales) for the selected rows."""
    pay, sc = [], []
    x = wl.x.values
    for r in rows_idx:
        p, s = O.dispatch_row(x[row_src[r]], wl.cfg.payload)
        pay.append(p)
        sc.append(s)
    return pay, sc


def _dispatch_combine_compare(wl, o, p, x, full_check, sample_rows=1024,
                              sample_tokens=256):
    """Given identical routing on both sides (o: oracle route, p: GPU plan),
    compare dispatch, fixture and combine."""
    cfg = wl.cfg
    cap = O.rows_capacity(cfg.T, cfg.E, cfg.k, cfg.pad)
    o_tok, o_src = O.assign_slots(o["topk_idx"], o["offsets"], cfg.E, cap)
    d = moe.dispatch(x, p, payload="fp8" if cfg.payload == "fp8" else "same")
    sigma_d = to_dev(wl.sigma)
    y = moe.expert_fixture(d, p, sigma_d, y_dtype=torch_dtype(cfg.y_dtype))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(d["tok_row"]), o_tok)
    assert np.array_equal(to_host(d["row_src"]), o_src)

    valid = np.nonzero(o_src >= 0)[0]
    rng = np.random.default_rng(0)
    if full_check or len(valid) <= sample_rows:
        rsel = valid
    else:
        # random rows plus the first and last row of every expert segment
        firsts = o["offsets"][:-1][o["counts"] > 0]
        lasts = (o["offsets"][:-1] + o["counts"] - 1)[o["counts"] > 0]
        rsel = np.unique(np.concatenate(
            [rng.choice(valid, sample_rows, replace=False), firsts, lasts]))
    ridx = torch.from_numpy(rsel.astype(np.int64)).cuda()
    g_rows = to_host(d["rows"][ridx])
    g_sc = to_host(d["row_scales"][ridx]) if cfg.payload == "fp8" else None
    g_y = to_host(y[ridx])
    pay, sc = _oracle_rows(wl, o_src, rsel)
    for i, r in enumerate(rsel):
        assert np.array_equal(g_rows[i], pay[i]), f"row {r}"
        if g_sc is not None:
            assert np.array_equal(g_sc[i], sc[i]), f"scales of row {r}"
        e = O.expert_of_row(o["offsets"], r)
        oy = O.expert_fixture_row(pay[i], sc[i], wl.sigma[e], cfg.payload,
                                  cfg.y_dtype)
        assert np.array_equal(g_y[i], oy), f"fixture row {r}"

    # combine, with the oracle's weights on both sides
    w_d = to_dev(o["topk_w"])
    shared = to_dev(wl.shared) if wl.shared is not None else None
    resid = to_dev(wl.residual) if wl.residual is not None else None
    if resid is not None:
        res_out, rnr = moe.combine_residual(y, d["tok_row"], w_d, shared, resid)
    else:
        out = moe.combine_residual(y, d["tok_row"], w_d, shared, None,
                                   out_dtype=torch_dtype(cfg.y_dtype))
    torch.cuda.synchronize()
    if full_check or cfg.T <= sample_tokens:
        tsel = np.arange(cfg.T)
    else:
        tsel = np.unique(np.concatenate([rng.choice(cfg.T, sample_tokens,
                                                    replace=False),
                                         [0, cfg.T - 1]]))
    tidx = torch.from_numpy(tsel.astype(np.int64)).cuda()
    x_vals = wl.x.values
    routed = np.zeros((len(tsel), cfg.H))
    for i, t in enumerate(tsel):
        yrows = []
        for j in range(cfg.k):
            e = int(o["topk_idx"][t, j])
            pj, sj = O.dispatch_row(x_vals[t], cfg.payload)
            yr = O.expert_fixture_row(pj, sj, wl.sigma[e], cfg.payload,
                                      cfg.y_dtype)
            yrows.append(yr if cfg.y_dtype == "f32" else O.bf16_value(yr))
        routed[i] = O.combine_token(np.array(yrows), o["topk_w"][t])
    if resid is not None:
        sh = wl.shared.values[tsel] if wl.shared is not None else None
        o_res, o_rnr, o_exact = O.farskip_update(routed, sh,
                                                 wl.residual.values[tsel])
        err = check_bf16_close(to_host(res_out[tidx]), o_exact, what="residual")
        assert np.array_equal(to_host(rnr[tidx]), o_rnr)
        note(f"combine max|err| residual={err:.2e}")
    else:
        if cfg.y_dtype == "f32":
            check_f32_close(to_host(out[tidx]), routed, what="routed f32")
        else:
            err = check_bf16_close(to_host(out[tidx]), routed, what="routed")
            note(f"combine max|err| routed={err:.2e}")


def _dc_case(name, cfg, seed, full_check):
    note(f"dispatch/combine {name} seed={seed} T={cfg.T} H={cfg.H} E={cfg.E} "
         f"k={cfg.k} payload={cfg.payload}")
    wl = I.make_workload(cfg, seed)
    o = O.route(wl.x.values, wl.w_gate.values, wl.bias, cfg.k, cfg.pad)
    idx_d = to_dev(o["topk_idx"])
    p = moe.plan(idx_d, cfg.E, cfg.pad)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(p["counts"]), o["counts"])
    assert np.array_equal(to_host(p["offsets"]), o["offsets"])
    x = to_dev(wl.x)
    _dispatch_combine_compare(wl, o, p, x, full_check)


@pytest.mark.parametrize("name", list(SMALL))
def test_dispatch_combine_small(name):
    _dc_case(name, SMALL[name], 2, full_check=True)


@pytest.mark.parametrize("name", FULL)
def test_dispatch_combine_full(name):
    _dc_case(name, C[name], 0, full_check=False)
