"""Seeded synthetic inputs for the MoE route -> dispatch -> combine transform.

This module only draws random numbers and packs them into the dtypes a
workload names.  It performs none of the method's arithmetic (no gate, no
softmax, no top-k, no scan, no quantisation), so the oracle and the HIP path
can both be fed from it without sharing any of the computation under test.

Every tensor is drawn from ``numpy.random.default_rng([seed, tensor_id])``
(PCG64) as float32 and, where the workload is bf16, rounded to the nearest
bf16 (ties to even).  Tensor ids: x=1, gate weight=2, expert permutation=3,
expert scales=4, shared-expert output=5, residual=6.

There are five synthetic workloads (Tiny, Mixtral-8x7B-shaped, DeepSeek-V3
decode- and prefill-shaped, and a MoonEP-shaped skewed load).  The shapes come from the models the pages name:
Mixtral 8x7B and DeepSeek R1/V3 ("Efficient and Portable Mixture-of-Experts
Communication", Introduction) and MoonEP's ``Buffer(S, H, K, E, ...)``
example with H=768, K=8, E=384 and ``token_padding`` 128 ("MoonEP developer
guide", core API example and core configuration parameters).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

TID_X, TID_W, TID_PERM, TID_SIGMA, TID_SHARED, TID_RESID = 1, 2, 3, 4, 5, 6
TID_GRAD = 7
TID_WCODE, TID_WSCALE = 8, 9

# Zipf exponent of the skewed workload and the strength with which its
# log-probabilities enter the router logits.  0.17 gives a max/mean expert
# load of about 5-10 on the MoonEP-shaped workload (checked by a test).
ZIPF_S = 1.2
ZIPF_BETA = 0.17


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int
    H: int
    E: int
    k: int
    pad: int
    x_dtype: str          # "f32" | "bf16"   (gate weight has the same dtype)
    payload: str          # "f32" | "bf16" | "fp8"   dispatched row dtype
    y_dtype: str          # "f32" | "bf16"   expert output dtype
    expert: str           # "identity" | "scale"   test fixture expert
    residual: bool        # fused dual-residual update vs routed-only output
    zipf_bias: bool = False

    def with_shape(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", T=64, H=128, E=8, k=2, pad=1, x_dtype="f32",
                   payload="f32", y_dtype="f32", expert="identity",
                   residual=False),
    "mixtral": Config("mixtral", T=4096, H=4096, E=8, k=2, pad=128,
                      x_dtype="bf16", payload="bf16", y_dtype="bf16",
                      expert="scale", residual=False),
    "dsv3_decode": Config("dsv3_decode", T=128, H=7168, E=256, k=8, pad=128,
                          x_dtype="bf16", payload="bf16", y_dtype="bf16",
                          expert="scale", residual=True),
    "dsv3_prefill": Config("dsv3_prefill", T=16384, H=7168, E=256, k=8,
                           pad=128, x_dtype="bf16", payload="fp8",
                           y_dtype="bf16", expert="scale", residual=True),
    "moonep_skew": Config("moonep_skew", T=8192, H=768, E=384, k=8, pad=128,
                          x_dtype="bf16", payload="bf16", y_dtype="bf16",
                          expert="identity", residual=True, zipf_bias=True),
}
CONFIG_ORDER = ["tiny", "mixtral", "dsv3_decode", "dsv3_prefill", "moonep_skew"]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) of finite float32 values, as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _rng(seed: int, tid: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tid)])


def _normal(seed, tid, shape, std=1.0):
    a = _rng(seed, tid).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


@dataclasses.dataclass
class Tensor:
    """A host tensor in its storage dtype.  ``bits`` holds the raw storage
    (float32 array for f32, uint16 bf16 patterns for bf16); ``values`` is the
    exact float32 value of every element."""
    dtype: str
    bits: np.ndarray

    @property
    def values(self) -> np.ndarray:
        if self.dtype == "f32":
            return self.bits
        return bf16_bits_to_f32(self.bits)

    @property
    def shape(self):
        return self.bits.shape


def _pack(a: np.ndarray, dtype: str) -> Tensor:
    if dtype == "f32":
        return Tensor("f32", np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        return Tensor("bf16", f32_to_bf16_bits(a))
    raise ValueError(dtype)


@dataclasses.dataclass
class Workload:
    cfg: Config
    seed: int
    x: Tensor                      # [T, H]
    w_gate: Tensor                 # [E, H]
    bias: Optional[np.ndarray]     # [E] float32 or None
    sigma: np.ndarray              # [E] float32 expert-fixture scales
    shared: Optional[Tensor]       # [T, H] bf16 or None
    residual: Optional[Tensor]     # [T, H] bf16 or None


def zipf_bias(E: int, seed: int, s: float = ZIPF_S,
              beta: float = ZIPF_BETA) -> np.ndarray:
    """Per-expert router bias from a Zipf(s) law over a seeded expert
    permutation: expert e has rank r_e = 1 + position of e in the
    permutation and bias beta * log(r_e ** -s)."""
    perm = _rng(seed, TID_PERM).permutation(E)
    rank = np.empty(E, dtype=np.int64)
    rank[perm] = np.arange(1, E + 1)
    return (np.float32(-s * beta) * np.log(rank).astype(np.float32)).astype(
        np.float32)


def make_workload(cfg: Config, seed: int = 0, w_std: Optional[float] = None,
                  sigma_set=None) -> Workload:
    """Draw every input tensor of one workload.

    ``w_std`` overrides the gate-weight standard deviation (default 1/sqrt(H)).
    ``sigma_set`` draws the expert scales from a finite set instead of
    U[0.5, 1.5] (used by closed-form tests that want exact products).
    """
    T, H, E = cfg.T, cfg.H, cfg.E
    x = _pack(_normal(seed, TID_X, (T, H)), cfg.x_dtype)
    std = (1.0 / np.sqrt(H)) if w_std is None else w_std
    w = _pack(_normal(seed, TID_W, (E, H), std), cfg.x_dtype)
    bias = zipf_bias(E, seed) if cfg.zipf_bias else None
    if cfg.expert == "identity":
        sigma = np.ones(E, dtype=np.float32)
    elif sigma_set is not None:
        sigma = np.asarray(sigma_set, dtype=np.float32)[
            _rng(seed, TID_SIGMA).integers(0, len(sigma_set), size=E)]
    else:
        sigma = _rng(seed, TID_SIGMA).uniform(0.5, 1.5, size=E).astype(
            np.float32)
    shared = residual = None
    if cfg.residual:
        shared = _pack(_normal(seed, TID_SHARED, (T, H), 0.1), "bf16")
        residual = _pack(_normal(seed, TID_RESID, (T, H)), "bf16")
    return Workload(cfg, seed, x, w, bias, sigma, shared, residual)


def integer_workload(cfg: Config, seed: int = 0, lo: int = -2,
                     hi: int = 2) -> Workload:
    """Small-integer x and gate weight: every partial sum of the gate is an
    exact integer in fp32 whatever the summation order, so the logits are
    exact on any hardware and top-k ties are frequent and exact."""
    base = make_workload(cfg, seed)
    rx = _rng(seed, 100 + TID_X).integers(lo, hi + 1, size=(cfg.T, cfg.H))
    rw = _rng(seed, 100 + TID_W).integers(lo, hi + 1, size=(cfg.E, cfg.H))
    base.x = _pack(rx.astype(np.float32), cfg.x_dtype)
    base.w_gate = _pack(rw.astype(np.float32), cfg.x_dtype)
    return base



def grad_tensor(seed: int, shape, dtype: str = "bf16", std: float = 1.0,
                stream: int = 0) -> Tensor:
    """Upstream gradient for the backward passes: N(0, std^2), rounded to
    ``dtype``.  ``stream`` separates several gradients of one seed."""
    return _pack(_normal(seed, TID_GRAD * 1000 + stream, tuple(shape), std),
                 dtype)


def expert_weights_fp8(seed: int, E: int, N: int, K: int,
                       experts=None):
    """Synthetic fp8 expert weights for the grouped GEMM: E4M3 codes [E, N, K]
    (uint8) with a random sign, exponent field uniform in 4..9 and random
    mantissa (magnitudes 2^-3 .. 7.5, never NaN), and block scales
    [E, N/128, K/128] float32 uniform in [0.5, 1.5] / sqrt(K).  With
    ``experts`` given, only those experts get random codes (drawn from a
    generator seeded by the expert id) and the others are zero."""
    codes = np.zeros((E, N, K), dtype=np.uint8)
    scales = (_rng(seed, TID_WSCALE).uniform(0.5, 1.5, size=(E, N // 128,
                                                             K // 128))
              / np.sqrt(K)).astype(np.float32)
    todo = range(E) if experts is None else experts
    for e in todo:
        g = _rng(seed, TID_WCODE * 100000 + int(e))
        sign = g.integers(0, 2, size=(N, K), dtype=np.uint8)
        expo = g.integers(4, 10, size=(N, K), dtype=np.uint8)
        mant = g.integers(0, 8, size=(N, K), dtype=np.uint8)
        codes[e] = (sign << 7) | (expo << 3) | mant
    return codes, scales
