"""GPU parity on seeded random shapes across the whole argument envelope.

Each configuration is drawn once from a fixed seed (half of the token and
expert counts log-uniform, half uniform over the upper range): T from 1 to
6000 tokens, H a multiple of 8 from 8 to 2048 (a multiple of 128 for fp8
payloads), 1 to 1024 experts (bf16 x above 512, as the C ABI requires), k
from 1 to min(16, E), pad from 1 to 128, x in bf16 or fp32, payload equal to
x or fp8, expert outputs in bf16 or fp32, with or without the dual residual
and a router bias.  Every configuration goes through the same checks as the
named shapes: route against the oracle (logits, exact top-k away from near
ties, counts and offsets, the route's own plan driving dispatch), then
dispatch / fixture / combine from the oracle's routing, element by element.
The same kind of draw drives the backward passes (combine and dispatch
backward against their fp64 definitions) and the fp8 grouped expert GEMM
(K and N multiples of 128, every routed row against the blocked oracle).
"""
import numpy as np
import pytest

import torch

from combine_router_gate_amd import inputs as I
from combine_router_gate_amd import moe
from oracle import moe_oracle as O
from _gpu_common import check_bf16_close, note, to_dev, to_host, torch_dtype
from test_gpu_backward import U, _combine_backward_case, _forward
from test_gpu_gemm import _gemm_case
from test_gpu_parity import _dc_case, _route_case

pytestmark = pytest.mark.gpu


def _draw(rng):
    while True:
        x_dtype = "bf16" if rng.random() < 0.7 else "f32"
        if rng.random() < 0.5:
            E = int(np.exp(rng.uniform(0.0, np.log(1024.0))).round())
        else:
            E = int(rng.integers(64, 1025))
        E = max(1, min(1024, E))
        if x_dtype == "f32" and E > 512:
            continue
        k = int(rng.integers(1, min(16, E) + 1))
        if rng.random() < 0.5:
            T = int(np.exp(rng.uniform(0.0, np.log(6000.0))).round())
        else:
            T = int(rng.integers(500, 6001))
        payload = "fp8" if rng.random() < 0.35 else x_dtype
        if payload == "fp8":
            H = 128 * int(rng.integers(1, 17))
        else:
            H = 8 * int(rng.integers(1, 257))
        if T * k > 40000 or T * H * E > 4e9:
            continue
        pad = int(rng.choice([1, 2, 3, 8, 16, 37, 64, 128]))
        y_dtype = "bf16" if rng.random() < 0.6 else "f32"
        return I.Config(f"rand_t{T}_h{H}_e{E}_k{k}", T=T, H=H, E=E, k=k,
                        pad=pad, x_dtype=x_dtype, payload=payload,
                        y_dtype=y_dtype,
                        expert="scale" if rng.random() < 0.5 else "identity",
                        residual=bool(rng.random() < 0.5),
                        zipf_bias=bool(rng.random() < 0.3))


_rng = np.random.default_rng(20261203)
CASES = [_draw(_rng) for _ in range(32)]


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_random_route(cfg):
    _route_case(cfg.name, cfg, 5)


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_random_dispatch_combine(cfg):
    _dc_case(cfg.name, cfg, 6, full_check=True)


@pytest.mark.parametrize("cfg", CASES[:16], ids=[c.name for c in CASES[:16]])
def test_random_combine_backward(cfg):
    _combine_backward_case(cfg.name, cfg, 8)


@pytest.mark.parametrize("cfg", CASES[16:], ids=[c.name for c in CASES[16:]])
def test_random_dispatch_backward(cfg):
    out_dtype = "f32" if cfg.T % 2 else "bf16"
    note(f"dispatch backward {cfg.name} out={out_dtype}")
    wl, o, d, y, o_tok, o_src = _forward(cfg, 9)
    cap = d["rows"].shape[0]
    G = I.grad_tensor(9, (cap, cfg.H), stream=1)
    gx = moe.dispatch_backward(to_dev(G), d["tok_row"],
                               out_dtype=torch_dtype(out_dtype))
    torch.cuda.synchronize()
    exact = O.dispatch_backward(G.values, o_tok)
    bound = cfg.k * U * O.dispatch_backward(np.abs(G.values), o_tok)
    got = to_host(gx)
    if out_dtype == "f32":
        assert (np.abs(got.astype(np.float64) - exact) <= bound + 1e-38).all()
    else:
        check_bf16_close(got, exact, tol=bound + 1e-38, what="grad_x")


def _draw_gemm(rng):
    while True:
        if rng.random() < 0.5:
            E = int(np.exp(rng.uniform(0.0, np.log(1024.0))).round())
        else:
            E = int(rng.integers(64, 1025))
        E = max(1, min(1024, E))
        k = int(rng.integers(1, min(8, E) + 1))
        T = int(rng.integers(1, 3001))
        K = 128 * int(rng.integers(1, 17))
        N = 128 * int(rng.integers(1, 9))
        if T * k * K * N > 4e9:
            continue
        pad = int(rng.choice([1, 8, 16, 64, 128, 256]))
        cfg = I.CONFIGS["dsv3_prefill"].with_shape(
            name=f"gemm_t{T}_k{K}_n{N}_e{E}", T=T, H=K, E=E, k=k, pad=pad,
            zipf_bias=bool(rng.random() < 0.3))
        return cfg, N, "bf16" if rng.random() < 0.6 else "f32"


_grng = np.random.default_rng(20261204)
GEMM_CASES = [_draw_gemm(_grng) for _ in range(12)]


@pytest.mark.parametrize("case", GEMM_CASES,
                         ids=[c[0].name for c in GEMM_CASES])
def test_random_expert_gemm(case):
    cfg, N, ydt = case
    _gemm_case(cfg.name, cfg, N, ydt, seed=33)
