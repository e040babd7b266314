"""GPU parity of the backward passes and of the FarSkip split form, through
the C ABI.

* moe_combine_backward: grad_y within one rounding of the exact w * g,
  grad_w within the summation bound of the fp64 oracle.
* moe_dispatch_backward: grad_x within the summation bound of the fp64 sum.
* moe_farskip_aux + residual-only moe_combine_residual: bit-identical to the
  fused dual-residual call, in place and out of place.
The routing plan is the oracle's (handed to the GPU through moe_plan), and
the expert outputs y that the oracle differentiates are the oracle's own,
recomputed from x; the GPU's y is first checked equal to them.
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
U = 2.0 ** -24          # unit roundoff of fp32

SMALL = {
    "decode": C["dsv3_decode"],
    "mixtral_s": C["mixtral"].with_shape(T=300, H=512),
    "f32_y": C["tiny"].with_shape(T=130, H=256, E=20, k=3, pad=5),
    "e512_k16": C["moonep_skew"].with_shape(T=100, H=64, E=512, k=16, pad=8,
                                            zipf_bias=False),
    "fp8_rows": C["dsv3_prefill"].with_shape(T=200, H=512, payload="fp8"),
    "h8_k1": C["mixtral"].with_shape(T=65, H=8, E=24, k=1, pad=1),
}


def _forward(cfg, seed):
    """Oracle routing on the GPU plan; GPU dispatch + fixture."""
    wl = I.make_workload(cfg, seed)
    o = O.route(wl.x.values, wl.w_gate.values, wl.bias, cfg.k, cfg.pad)
    p = moe.plan(to_dev(o["topk_idx"]), cfg.E, cfg.pad)
    x = to_dev(wl.x)
    d = moe.dispatch(x, p, payload="fp8" if cfg.payload == "fp8" else "same")
    y = moe.expert_fixture(d, p, to_dev(wl.sigma),
                           y_dtype=torch_dtype(cfg.y_dtype))
    torch.cuda.synchronize()
    cap = O.rows_capacity(cfg.T, cfg.E, cfg.k, cfg.pad)
    o_tok, o_src = O.assign_slots(o["topk_idx"], o["offsets"], cfg.E, cap)
    assert np.array_equal(to_host(d["tok_row"]), o_tok)
    return wl, o, d, y, o_tok, o_src


def _oracle_y_rows(wl, o, o_src, rows):
    """Oracle expert outputs (float64 values of their storage) of the given
    rows of the expert-major buffer."""
    cfg = wl.cfg
    out = np.zeros((len(rows), cfg.H))
    for i, r in enumerate(rows):
        if o_src[r] < 0:
            continue
        pay, sc = O.dispatch_row(wl.x.values[o_src[r]], cfg.payload)
        e = O.expert_of_row(o["offsets"], r)
        yr = O.expert_fixture_row(pay, sc, wl.sigma[e], cfg.payload,
                                  cfg.y_dtype)
        out[i] = yr if cfg.y_dtype == "f32" else O.bf16_value(yr)
    return out


def _check_grad_y(gpu_bits, exact):
    """One product rounded to fp32, then to bf16: within half a bf16 ulp of
    the exact value plus one fp32 rounding."""
    return check_bf16_close(gpu_bits, exact, tol=U * np.abs(exact) + 1e-38,
                            what="grad_y")


def _check_grad_w(gpu, exact, g, yrows, H):
    """fp32 dot product over H: a lane sums at most H/(64 w) + 8 products in
    order (w waves share the token), then a 6-level lane butterfly and an
    in-order sum of the w partials; for the w the launcher picks this is at
    most H/64 + 8 roundings on the way, so |err| <= (H/64 + 8) u
    sum|g_h y_h|."""
    mag = np.abs(g[:, None, :] * yrows).sum(axis=2)
    bound = (H / 64 + 8) * U * mag + 1e-30
    err = np.abs(np.asarray(gpu, np.float64) - exact)
    assert (err <= bound).all(), (err.max(), np.argwhere(err > bound)[:5])


def _combine_backward_case(name, cfg, seed, tokens=None):
    note(f"combine backward {name} seed={seed} T={cfg.T} H={cfg.H} E={cfg.E} "
         f"k={cfg.k} y={cfg.y_dtype}")
    wl, o, d, y, o_tok, o_src = _forward(cfg, seed)
    g = I.grad_tensor(seed, (cfg.T, cfg.H))
    gy, gw = moe.combine_backward(to_dev(g), y, d["tok_row"], to_dev(o["topk_w"]))
    torch.cuda.synchronize()
    tsel = np.arange(cfg.T) if tokens is None else tokens
    k = cfg.k
    rows = o_tok[tsel].ravel()
    yr = _oracle_y_rows(wl, o, o_src, rows)
    rsel = torch.from_numpy(rows.astype(np.int64)).cuda()
    # the GPU's y is the oracle's y: differentiating the same function
    if cfg.y_dtype == "f32":
        assert np.array_equal(to_host(y[rsel]).astype(np.float64), yr)
    else:
        assert np.array_equal(O.bf16_value(to_host(y[rsel])), yr)
    gv = g.values[tsel]
    sub_tok = np.arange(len(rows), dtype=np.int64).reshape(len(tsel), k)
    o_gy, o_gw = O.combine_backward(gv, yr, sub_tok, o["topk_w"][tsel],
                                    len(rows))
    _check_grad_y(to_host(gy[rsel]), o_gy)
    tidx = torch.from_numpy(tsel.astype(np.int64)).cuda()
    _check_grad_w(to_host(gw[tidx]), o_gw, gv.astype(np.float64),
                  yr.reshape(len(tsel), k, cfg.H), cfg.H)
    if tokens is None:
        # rows that no slot references are never written (zeros from the
        # wrapper's allocation)
        unref = np.nonzero(o_src < 0)[0]
        if len(unref):
            u = torch.from_numpy(unref.astype(np.int64)).cuda()
            assert not to_host(gy[u]).any()


@pytest.mark.parametrize("name", list(SMALL))
def test_combine_backward_small(name):
    _combine_backward_case(name, SMALL[name], 11)


def test_combine_backward_prefill_sampled():
    cfg = C["dsv3_prefill"]
    rng = np.random.default_rng(3)
    toks = np.unique(np.concatenate([rng.choice(cfg.T, 96, replace=False),
                                     [0, cfg.T - 1]]))
    _combine_backward_case("dsv3_prefill", cfg, 0, tokens=toks)


@pytest.mark.parametrize("name,out_dtype", [("decode", "f32"),
                                            ("mixtral_s", "bf16"),
                                            ("e512_k16", "f32"),
                                            ("h8_k1", "bf16")])
def test_dispatch_backward(name, out_dtype):
    cfg = SMALL[name]
    note(f"dispatch backward {name} out={out_dtype}")
    wl, o, d, y, o_tok, o_src = _forward(cfg, 12)
    cap = d["rows"].shape[0]
    G = I.grad_tensor(12, (cap, cfg.H), stream=1)
    gx = moe.dispatch_backward(to_dev(G), d["tok_row"],
                               out_dtype=torch_dtype(out_dtype))
    torch.cuda.synchronize()
    exact = O.dispatch_backward(G.values, o_tok)
    mag = O.dispatch_backward(np.abs(G.values), o_tok)
    bound = cfg.k * U * mag
    got = to_host(gx)
    if out_dtype == "f32":
        err = np.abs(got.astype(np.float64) - exact)
        assert (err <= bound + 1e-38).all(), err.max()
    else:
        check_bf16_close(got, exact, tol=bound + 1e-38, what="grad_x")


def test_dispatch_backward_f32_rows_full_prefill_sampled():
    """At the prefill shape with fp32 gradient rows: sampled tokens."""
    cfg = C["dsv3_prefill"]
    note("dispatch backward dsv3_prefill f32 rows, sampled")
    wl = I.make_workload(cfg, 0)
    o = O.route(wl.x.values, wl.w_gate.values, wl.bias, cfg.k, cfg.pad)
    cap = O.rows_capacity(cfg.T, cfg.E, cfg.k, cfg.pad)
    o_tok, _ = O.assign_slots(o["topk_idx"], o["offsets"], cfg.E, cap)
    G = I.grad_tensor(0, (cap, cfg.H), dtype="f32", stream=2)
    tok_row = to_dev(o_tok.astype(np.int32))
    gx = moe.dispatch_backward(to_dev(G), tok_row, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    tsel = np.unique(np.concatenate([rng.choice(cfg.T, 128, replace=False),
                                     [0, cfg.T - 1]]))
    rows = o_tok[tsel].ravel()
    sub_tok = np.arange(len(rows)).reshape(len(tsel), cfg.k)
    Gs = G.values[rows]
    exact = O.dispatch_backward(Gs, sub_tok)
    mag = O.dispatch_backward(np.abs(Gs), sub_tok)
    got = to_host(gx[torch.from_numpy(tsel).cuda()]).astype(np.float64)
    assert (np.abs(got - exact) <= cfg.k * U * mag + 1e-38).all()


# ----------------------------------------------------------- FarSkip split

SPLIT = {"decode": SMALL["decode"],
         "moonep_s": C["moonep_skew"].with_shape(T=517),
         "fp8_rows": SMALL["fp8_rows"]}


@pytest.mark.parametrize("name,with_shared", [("decode", True),
                                              ("moonep_s", False),
                                              ("fp8_rows", True)])
def test_farskip_split_equals_fused(name, with_shared):
    cfg = SPLIT[name]
    note(f"farskip split {name} shared={with_shared}")
    wl, o, d, y, o_tok, o_src = _forward(cfg, 13)
    res = to_dev(wl.residual)
    sh = to_dev(wl.shared) if with_shared else None
    w = to_dev(o["topk_w"])
    f_res, f_rnr = moe.combine_residual(y, d["tok_row"], w, sh, res)
    rnr = moe.farskip_aux(sh, res)
    s_res = moe.combine_main_residual(y, d["tok_row"], w, sh, res)
    torch.cuda.synchronize()
    assert torch.equal(rnr.view(torch.int16), f_rnr.view(torch.int16))
    assert torch.equal(s_res.view(torch.int16), f_res.view(torch.int16))
    # aux against the oracle, exact
    sv = wl.shared.values if with_shared else None
    _, o_rnr, _ = O.farskip_update(np.zeros((cfg.T, cfg.H)), sv,
                                   wl.residual.values)
    assert np.array_equal(to_host(rnr), o_rnr)
    # in place: the auxiliary stream first (it reads residual), then the
    # main stream overwrites residual
    res2 = res.clone()
    rnr2 = moe.farskip_aux(sh, res2)
    out2 = moe.combine_main_residual(y, d["tok_row"], w, sh, res2,
                                     in_place=True)
    torch.cuda.synchronize()
    assert out2.data_ptr() == res2.data_ptr()
    assert torch.equal(res2.view(torch.int16), f_res.view(torch.int16))
    assert torch.equal(rnr2.view(torch.int16), f_rnr.view(torch.int16))


def test_farskip_aux_empty():
    r = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    assert moe.farskip_aux(None, r).shape == (0, 256)


@pytest.mark.parametrize("name", ["decode", "mixtral_s"])
def test_backward_deterministic(name):
    """Both backward passes give the same bits on every call (fixed
    summation orders, no atomics)."""
    cfg = SMALL[name]
    note(f"backward determinism {name}")
    wl, o, d, y, o_tok, o_src = _forward(cfg, 13)
    g = to_dev(I.grad_tensor(13, (cfg.T, cfg.H)))
    w = to_dev(o["topk_w"])
    cap = d["rows"].shape[0]
    G = to_dev(I.grad_tensor(13, (cap, cfg.H), stream=1))
    first = None
    for _ in range(3):
        gy, gw = moe.combine_backward(g, y, d["tok_row"], w)
        gx = moe.dispatch_backward(G, d["tok_row"])
        torch.cuda.synchronize()
        cur = (gy.view(torch.int16).clone(), gw.view(torch.int32).clone(),
               gx.view(torch.int32).clone())
        if first is None:
            first = cur
        else:
            assert all(torch.equal(a, b) for a, b in zip(first, cur))
