"""moe_route_dispatch_one_launch (gate partial sums, top-k, plan and scatter
in one kernel with two grid-wide waits) through the C ABI, against the
oracle: logits within tolerance, the top-k exact on the kernel's own logits,
a valid stable plan, sampled payload rows; the exact plan on integer inputs;
and the same rows as moe_route_dispatch whenever both chose the same
experts.  Consecutive calls of different shapes check that the wait
counters carry over from call to call; 12 seeded random configurations
(1-256 tokens, 1-512 experts, k up to 16, bf16 or fp8 payloads, router bias)
cover the envelope."""
import numpy as np
import pytest
import torch

from combine_router_gate_amd import inputs as I
from combine_router_gate_amd import moe
from oracle import moe_oracle as O
from _gpu_common import (LOGIT_TOL, check_plan_valid, check_topk_own_logits,
                         note, to_dev, to_host)
from test_gpu_route_dispatch import _sampled_rows

pytestmark = pytest.mark.gpu

C = I.CONFIGS
CASES = {
    "decode": C["dsv3_decode"],
    "decode_fp8": C["dsv3_decode"].with_shape(payload="fp8"),
    "t1": C["dsv3_decode"].with_shape(T=1, H=2048),
    "t256_e512_k16": C["moonep_skew"].with_shape(T=256, H=512, E=512, k=16,
                                                 pad=8, zipf_bias=False),
    "t255_e384_bias": C["moonep_skew"].with_shape(T=255),
    "t97_e20_h64": C["dsv3_decode"].with_shape(T=97, H=64, E=20, k=3, pad=2),
    "t130_e100_fp8": C["dsv3_decode"].with_shape(T=130, H=256, E=100, k=4,
                                                 pad=3, payload="fp8"),
}


def _payload(cfg):
    return "fp8" if cfg.payload == "fp8" else "same"


@pytest.mark.parametrize("name", list(CASES))
def test_one_launch_against_oracle(name):
    cfg = CASES[name]
    note(f"one_launch {name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} "
         f"payload={cfg.payload}")
    wl = I.make_workload(cfg, 7)
    x, w = to_dev(wl.x), to_dev(wl.w_gate)
    b = to_dev(wl.bias) if wl.bias is not None else None
    p, d = moe.route_dispatch(x, w, cfg.k, cfg.pad, bias=b,
                              payload=_payload(cfg), want_logits=True,
                              one_launch=True)
    p2, d2 = moe.route_dispatch(x, w, cfg.k, cfg.pad, bias=b,
                                payload=_payload(cfg), want_logits=True)
    torch.cuda.synchronize()
    o = O.route(wl.x.values, wl.w_gate.values, wl.bias, cfg.k, cfg.pad)
    gl = to_host(p["logits"])
    assert np.abs(gl.astype(np.float64) - o["logits"]).max() <= LOGIT_TOL
    gi = to_host(p["topk_idx"])
    check_topk_own_logits(gi, to_host(p["topk_w"]), gl, cfg.k)
    check_plan_valid(gi, to_host(p["counts"]), to_host(p["offsets"]),
                     to_host(d["tok_row"]), to_host(d["row_src"]), cfg.E,
                     cfg.pad)
    _sampled_rows(wl, d, cfg)
    # the same choices as the three-launch path give the same plan and rows
    if np.array_equal(gi, to_host(p2["topk_idx"])):
        for key in ("counts", "offsets"):
            assert np.array_equal(to_host(p[key]), to_host(p2[key])), key
        for key in ("row_src", "tok_row"):
            assert np.array_equal(to_host(d[key]), to_host(d2[key])), key
        valid = torch.from_numpy(
            np.nonzero(to_host(d["row_src"]) >= 0)[0]).cuda()
        assert np.array_equal(to_host(d["rows"][valid]).view(np.uint8),
                              to_host(d2["rows"][valid]).view(np.uint8))
        np.testing.assert_allclose(to_host(p["topk_w"]),
                                   to_host(p2["topk_w"]), rtol=1e-5,
                                   atol=1e-7)


@pytest.mark.parametrize("name", ["decode", "t256_e512_k16", "t97_e20_h64"])
def test_one_launch_integer_inputs_equal_oracle_plan(name):
    """Exact logits: the routing and the whole plan equal the oracle's."""
    cfg = CASES[name]
    note(f"one_launch integer {name}")
    wl = I.integer_workload(cfg, 4)
    x, w = to_dev(wl.x), to_dev(wl.w_gate)
    p, d = moe.route_dispatch(x, w, cfg.k, cfg.pad, payload=_payload(cfg),
                              one_launch=True)
    torch.cuda.synchronize()
    o = O.route(wl.x.values, wl.w_gate.values, None, cfg.k, cfg.pad)
    assert np.array_equal(to_host(p["topk_idx"]), o["topk_idx"])
    assert np.array_equal(to_host(p["counts"]), o["counts"])
    assert np.array_equal(to_host(p["offsets"]), o["offsets"])
    cap = O.rows_capacity(cfg.T, cfg.E, cfg.k, cfg.pad)
    o_tok, o_src = O.assign_slots(o["topk_idx"], o["offsets"], cfg.E, cap)
    assert np.array_equal(to_host(d["tok_row"]), o_tok)
    assert np.array_equal(to_host(d["row_src"]), o_src)
    _sampled_rows(wl, d, cfg, n=256)


def test_one_launch_back_to_back_shapes():
    """Calls of different grids queued without synchronisation in between,
    interleaved with other launches: each must still wait for its own grid
    only (the counters' running total is kept per call on the host)."""
    names = ["t1", "decode", "t256_e512_k16", "t1", "t97_e20_h64"]
    runs = []
    for i, name in enumerate(names):
        cfg = CASES[name]
        wl = I.integer_workload(cfg, 10 + i)
        x, w = to_dev(wl.x), to_dev(wl.w_gate)
        p, d = moe.route_dispatch(x, w, cfg.k, cfg.pad,
                                  payload=_payload(cfg), one_launch=True)
        moe.route(x, w, cfg.k, cfg.pad)          # another launch between
        runs.append((cfg, wl, p, d))
    note(f"one_launch back to back: {names}")
    torch.cuda.synchronize()
    for cfg, wl, p, d in runs:
        o = O.route(wl.x.values, wl.w_gate.values, None, cfg.k, cfg.pad)
        assert np.array_equal(to_host(p["topk_idx"]), o["topk_idx"])
        assert np.array_equal(to_host(p["offsets"]), o["offsets"])
        cap = O.rows_capacity(cfg.T, cfg.E, cfg.k, cfg.pad)
        o_tok, o_src = O.assign_slots(o["topk_idx"], o["offsets"], cfg.E, cap)
        assert np.array_equal(to_host(d["tok_row"]), o_tok)
        assert np.array_equal(to_host(d["row_src"]), o_src)


def test_one_launch_no_tokens():
    cfg = C["dsv3_decode"].with_shape(T=0, H=256, E=64, k=4, pad=8)
    x = torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((cfg.E, cfg.H), dtype=torch.bfloat16, device="cuda")
    p, d = moe.route_dispatch(x, w, cfg.k, cfg.pad, one_launch=True)
    torch.cuda.synchronize()
    assert (to_host(p["counts"]) == 0).all()
    assert (to_host(p["offsets"]) == 0).all()
    assert (to_host(d["row_src"]) == -1).all()


def _draw(rng):
    E = int(rng.integers(1, 513))
    k = int(rng.integers(1, min(16, E) + 1))
    T = int(rng.integers(1, 257))
    payload = "fp8" if rng.random() < 0.4 else "bf16"
    H = 128 * int(rng.integers(1, 17)) if payload == "fp8" \
        else 8 * int(rng.integers(1, 257))
    pad = int(rng.choice([1, 2, 8, 37, 128]))
    return I.Config(f"rand_t{T}_h{H}_e{E}_k{k}", T=T, H=H, E=E, k=k, pad=pad,
                    x_dtype="bf16", payload=payload, y_dtype="bf16",
                    expert="identity", residual=False,
                    zipf_bias=bool(rng.random() < 0.4))


_rng = np.random.default_rng(20261205)
RANDOM = [_draw(_rng) for _ in range(12)]


@pytest.mark.parametrize("cfg", RANDOM, ids=[c.name for c in RANDOM])
def test_one_launch_random_shapes(cfg):
    note(f"one_launch random {cfg.name} pad={cfg.pad} payload={cfg.payload}")
    wl = I.make_workload(cfg, 11)
    x, w = to_dev(wl.x), to_dev(wl.w_gate)
    b = to_dev(wl.bias) if wl.bias is not None else None
    p, d = moe.route_dispatch(x, w, cfg.k, cfg.pad, bias=b,
                              payload=_payload(cfg), want_logits=True,
                              one_launch=True)
    torch.cuda.synchronize()
    o = O.route(wl.x.values, wl.w_gate.values, wl.bias, cfg.k, cfg.pad)
    gl = to_host(p["logits"])
    assert np.abs(gl.astype(np.float64) - o["logits"]).max() <= LOGIT_TOL
    gi = to_host(p["topk_idx"])
    check_topk_own_logits(gi, to_host(p["topk_w"]), gl, cfg.k)
    check_plan_valid(gi, to_host(p["counts"]), to_host(p["offsets"]),
                     to_host(d["tok_row"]), to_host(d["row_src"]), cfg.E,
                     cfg.pad)
    _sampled_rows(wl, d, cfg)
