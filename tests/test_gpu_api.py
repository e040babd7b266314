"""GPU tests of the C ABI beyond the workload parity tests: fp8 code
boundaries, determinism, in-place residual update, empty inputs and errors
raised for invalid arguments with real device tensors."""
import numpy as np
import pytest
import torch

from combine_router_gate_amd import inputs as I
from combine_router_gate_amd import moe
from oracle import moe_oracle as O
from _gpu_common import note, to_dev, to_host

pytestmark = pytest.mark.gpu


def _e4m3_magnitudes():
    out = []
    for c in range(127):                     # all finite non-negative codes
        ef, mf = c >> 3, c & 7
        out.append(mf * 2.0 ** -9 if ef == 0 else (8 + mf) * 2.0 ** (ef - 10))
    return np.array(sorted(set(out)))


def _boundary_values_f32():
    """E4M3 values, the midpoints between neighbours, and the float32
    neighbours of both, all with |v| <= 448, both signs."""
    v = _e4m3_magnitudes()
    mids = (v[:-1] + v[1:]) / 2
    pts = np.concatenate([v, mids, [2.0 ** -10, 2.0 ** -11, 1e-6, 3e-3]]).astype(
        np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(0))
    allv = np.concatenate([pts, up, dn])
    allv = allv[np.abs(allv) <= 448]
    return np.concatenate([allv, -allv, np.array([0.0, -0.0], np.float32)])


def _blocks_with_unit_scale(vals, H):
    """Rows of H elements; each 128-block starts with 448 so its scale is
    exactly 1 and every other element is encoded as-is."""
    per_row = (H // 128) * 127
    T = -(-len(vals) // per_row)
    pad = np.zeros(T * per_row, np.float32)
    pad[:len(vals)] = vals
    blocks = pad.reshape(T, H // 128, 127)
    x = np.concatenate([np.full((T, H // 128, 1), 448.0, np.float32), blocks],
                       axis=2).reshape(T, H)
    return x


def _dispatch_identity(x_dev, T, H):
    idx = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
    p = moe.plan(idx, 1, 1)
    return moe.dispatch(x_dev, p, payload="fp8")


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_fp8_codes_every_boundary(src):
    """The E4M3 codes written by moe_dispatch equal the oracle's independent
    encoder on every code value, midpoint and float32 neighbour (fp32 x) and
    on every bf16 magnitude <= 448 (bf16 x)."""
    H = 1024
    if src == "f32":
        vals = _boundary_values_f32()
        x = _blocks_with_unit_scale(vals, H)
        x_dev = torch.from_numpy(x).cuda()
    else:
        bits = np.arange(0, 0x8000, dtype=np.uint32)
        f = (bits << 16).view(np.float32)
        f = f[np.isfinite(f) & (np.abs(f) <= 448)]
        vals = np.concatenate([f, -f])
        x = _blocks_with_unit_scale(vals, H)
        xb = I.f32_to_bf16_bits(x)
        assert np.array_equal(I.bf16_bits_to_f32(xb), x)   # exact in bf16
        x_dev = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    T = x.shape[0]
    note(f"fp8 boundary codes src={src} values={len(vals)} T={T}")
    d = _dispatch_identity(x_dev, T, H)
    torch.cuda.synchronize()
    rows, scales = to_host(d["rows"]), to_host(d["row_scales"])
    for t in range(T):
        codes, s = O.quantize_row_e4m3(x[t])
        assert (s == 1.0).all()
        assert np.array_equal(scales[t], s), t
        bad = np.nonzero(rows[t] != codes)[0]
        assert bad.size == 0, (t, x[t][bad[:5]], rows[t][bad[:5]], codes[bad[:5]])


def test_determinism_bit_identical():
    """Two runs of the whole chain give bit-identical outputs (no float
    atomics; fixed slot order)."""
    cfg = I.CONFIGS["moonep_skew"].with_shape(T=777)
    wl = I.make_workload(cfg, 5)
    x, w = to_dev(wl.x), to_dev(wl.w_gate)
    b = to_dev(wl.bias)
    outs = []
    for _ in range(2):
        p = moe.route(x, w, cfg.k, cfg.pad, bias=b)
        d = moe.dispatch(x, p)
        y = moe.expert_fixture(d, p, to_dev(wl.sigma))
        res, rnr = moe.combine_residual(y, d["tok_row"], p["topk_w"],
                                        to_dev(wl.shared), to_dev(wl.residual))
        torch.cuda.synchronize()
        outs.append([to_host(t) for t in (p["topk_idx"], p["topk_w"],
                                          p["counts"], p["offsets"],
                                          d["tok_row"], d["row_src"], res, rnr)])
    for a, b2 in zip(*outs):
        assert np.array_equal(a, b2)


def test_inplace_residual_matches():
    cfg = I.CONFIGS["dsv3_decode"].with_shape(T=96, H=512, E=64, k=6, pad=16)
    wl = I.make_workload(cfg, 7)
    x = to_dev(wl.x)
    p = moe.route(x, to_dev(wl.w_gate), cfg.k, cfg.pad)
    d = moe.dispatch(x, p)
    y = moe.expert_fixture(d, p, to_dev(wl.sigma))
    sh, res = to_dev(wl.shared), to_dev(wl.residual)
    ref_out, ref_rnr = moe.combine_residual(y, d["tok_row"], p["topk_w"], sh, res)
    res2 = res.clone()
    out2, rnr2 = moe.combine_residual(y, d["tok_row"], p["topk_w"], sh, res2,
                                      in_place=True)
    torch.cuda.synchronize()
    assert out2.data_ptr() == res2.data_ptr()
    assert torch.equal(out2, ref_out) and torch.equal(rnr2, ref_rnr)


def test_empty_tokens():
    E, k, pad = 16, 2, 4
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.randn((E, 64), device="cuda").bfloat16()
    p = moe.route(x, w, k, pad)
    torch.cuda.synchronize()
    assert (p["counts"] == 0).all() and (p["offsets"] == 0).all()
    cap = 50                                    # >= E*(pad-1) = 48
    d = moe.dispatch(x, p, capacity=cap)
    torch.cuda.synchronize()
    assert (d["row_src"] == -1).all()          # every row is unused


def test_single_token_and_full_topk():
    cfg = I.CONFIGS["mixtral"].with_shape(T=1, H=256, E=8, k=8, pad=3)
    wl = I.make_workload(cfg, 2)
    x = to_dev(wl.x)
    p = moe.route(x, to_dev(wl.w_gate), cfg.k, cfg.pad)
    d = moe.dispatch(x, p)
    torch.cuda.synchronize()
    o = O.route(wl.x.values, wl.w_gate.values, None, cfg.k, cfg.pad)
    assert sorted(to_host(p["topk_idx"])[0].tolist()) == list(range(8))
    assert np.array_equal(to_host(p["offsets"]), o["offsets"])
    cap = O.rows_capacity(1, 8, 8, 3)
    tr, rs = O.assign_slots(o["topk_idx"], o["offsets"], 8, cap)
    # the GPU's own routing may order the 8 experts differently only at ties;
    # the slot of expert e is offsets[e] either way
    g_idx, g_tr = to_host(p["topk_idx"])[0], to_host(d["tok_row"])[0]
    assert all(g_tr[j] == o["offsets"][g_idx[j]] for j in range(8))


def test_errors_raise():
    x = torch.randn((10, 64), device="cuda").bfloat16()
    w = torch.randn((8, 64), device="cuda").bfloat16()
    with pytest.raises(moe.MoEError, match="SHAPE"):
        moe.route(x, w, 9, 1)                        # k > E
    p = moe.route(x, w, 2, 4)
    with pytest.raises(moe.MoEError, match="CAPACITY"):
        moe.dispatch(x, p, capacity=10 * 2 + 8 * 3 - 1)
    with pytest.raises(moe.MoEError, match="SHAPE"):
        moe.dispatch(x, p, payload="fp8")            # H % 128 != 0
    y = torch.empty((100, 64), dtype=torch.bfloat16, device="cuda")
    d = moe.dispatch(x, p)
    res = torch.zeros((10, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoEError, match="ALIAS"):
        moe.moe_combine_residual(y, d["tok_row"], p["topk_w"], None, res, res,
                                 res, None)           # rnr aliases residual
    torch.cuda.synchronize()


def test_route_nonfinite_weight_stays_in_its_logit():
    """An infinite gate weight inside one hidden range: that expert's logit
    is +inf (the fp64 oracle's value) and every other logit stays finite and
    within tolerance.  H = 192 over three 64-wide ranges makes each range one
    step, so the split gate runs a step past every range; weights outside a
    range must not meet that step's zero x as 0 * inf = NaN."""
    cfg = I.CONFIGS["dsv3_decode"].with_shape(T=64, H=192, E=64, k=4, pad=8)
    note("route with an infinite gate weight, T=64 H=192 E=64")
    wl = I.make_workload(cfg, 2)
    x = wl.x.values.copy()
    x[:, 100] = 1.0
    w = wl.w_gate.values.copy()
    w[5, 100] = np.inf
    xb = I._pack(x, "bf16")
    wb = I._pack(w, "bf16")
    p = moe.route(to_dev(xb), to_dev(wb), cfg.k, cfg.pad, want_logits=True)
    torch.cuda.synchronize()
    gl = to_host(p["logits"]).astype(np.float64)
    o = O.gate_logits(xb.values, wb.values)
    assert np.isposinf(o[:, 5]).all()
    assert np.isposinf(gl[:, 5]).all(), gl[:, 5][:8]
    rest = np.delete(np.arange(cfg.E), 5)
    assert np.isfinite(gl[:, rest]).all()
    assert np.abs(gl[:, rest] - o[:, rest]).max() <= 1e-4
