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
"""
import numpy as np
import pytest

from combine_router_gate_amd import inputs as I
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
