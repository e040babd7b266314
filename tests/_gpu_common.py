"""Shared helpers of the GPU parity tests: host <-> device conversion and
the comparison rules.  The oracle only ever receives generator inputs (or
its own results); GPU outputs are compared against it, never fed to it."""
import numpy as np
import torch

from combine_router_gate_amd import inputs as I
from oracle import moe_oracle as O

# Absolute bound on |GPU logit - fp64 logit|.  Logits are O(1); fp32
# accumulation of H <= 8192 products of O(1/sqrt(H)) terms errs by a few
# 1e-6, so 1e-4 leaves ample margin while still catching a dropped term.
LOGIT_TOL = 1e-4


def note(msg: str):
    print(f"[case] {msg}", flush=True)


def to_dev(t) -> torch.Tensor:
    if isinstance(t, I.Tensor):
        if t.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(t.bits)).cuda()
        return torch.from_numpy(
            np.ascontiguousarray(t.bits).view(np.int16)).view(
                torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(t)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    """Storage bits on the host: uint16 for bf16, raw for other dtypes."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def topk_audit(gpu_idx, gpu_w, oracle_logits, gpu_logits, k):
    """Compare the GPU's top-k with the oracle's.

    The choice is unique where the oracle's gap between the k-th and
    (k+1)-th logit exceeds twice the logit tolerance: there the sets must be
    equal, and the order must be equal wherever consecutive chosen logits are
    more than that apart.  Elsewhere (a near tie) the GPU's set must be valid:
    distinct experts whose oracle logits all lie within 2*LOGIT_TOL of the
    k-th largest.  Weights: with measured logit error d, every renormalised
    weight is within 2*d (+ fp32 rounding) of the oracle's.
    Returns the number of near-tie tokens."""
    l = np.asarray(oracle_logits)
    T, E = l.shape
    o_idx, o_w = O.select_topk(l, k)
    srt = -np.sort(-l, axis=1)
    gap = srt[:, k - 1] - (srt[:, k] if k < E else -np.inf)
    clear = gap > 2 * LOGIT_TOL
    gi = np.asarray(gpu_idx)
    assert ((gi >= 0) & (gi < E)).all()
    assert (np.sort(gi, axis=1)[:, 1:] != np.sort(gi, axis=1)[:, :-1]).all()
    same_set = (np.sort(gi, axis=1) == np.sort(o_idx, axis=1)).all(axis=1)
    bad = clear & ~same_set
    assert not bad.any(), f"top-k sets differ on clear tokens {np.nonzero(bad)[0][:10]}"
    # order inside the chosen set
    sel = np.take_along_axis(l, o_idx.astype(np.int64), axis=1)
    adj_clear = np.diff(-sel, axis=1) > 2 * LOGIT_TOL  # [T, k-1]
    for t in np.nonzero(clear)[0]:
        if k == 1 or adj_clear[t].all():
            assert (gi[t] == o_idx[t]).all(), t
    # near ties: validity
    near = ~clear
    for t in np.nonzero(near)[0]:
        assert (l[t, gi[t]] >= srt[t, k - 1] - 2 * LOGIT_TOL).all(), t
    # weights
    d = float(np.abs(np.asarray(gpu_logits, dtype=np.float64) - l).max()) \
        if gpu_logits is not None else LOGIT_TOL
    wt = 2 * d + 2e-6
    same_seq = (gi == o_idx).all(axis=1)
    gw = np.asarray(gpu_w, dtype=np.float64)
    err = np.abs(gw[same_seq] - o_w[same_seq].astype(np.float64))
    assert err.size == 0 or err.max() <= wt, (err.max(), wt)
    assert np.abs(gw.sum(axis=1) - 1.0).max() <= 1e-5
    return int(near.sum())


def check_bf16_close(gpu_bits, exact64, tol=1e-2, what=""):
    """bf16 outputs: |g - o*| <= tol + half a bf16 ulp of o*, where o* is the
    oracle's value before its final rounding (the bound "1e-2 absolute" on
    top of the one unavoidable rounding to bf16)."""
    g = O.bf16_value(gpu_bits)
    o = np.asarray(exact64, dtype=np.float64)
    _, e = np.frexp(o)
    half_ulp = np.ldexp(1.0, np.maximum(e, -125) - 9)
    err = np.abs(g - o)
    bad = err > tol + half_ulp
    assert not bad.any(), (what, err.max(), np.argwhere(bad)[:5])
    return float(err.max())


def check_f32_close(gpu, exact64, what=""):
    """fp32 outputs: |g - o| <= 1e-5 |o| + 1e-6."""
    g = np.asarray(gpu, dtype=np.float64)
    o = np.asarray(exact64, dtype=np.float64)
    bad = np.abs(g - o) > 1e-5 * np.abs(o) + 1e-6
    assert not bad.any(), (what, np.abs(g - o).max(), np.argwhere(bad)[:5])


def order_keys(logits_f32) -> np.ndarray:
    """Order-preserving integer key of float32 values (larger value, larger
    key; -0 ranks just below +0), as int64."""
    u = np.ascontiguousarray(logits_f32, dtype=np.float32).view(
        np.uint32).astype(np.int64)
    neg = (u & 0x80000000) != 0
    return np.where(neg, (~u) & 0xFFFFFFFF, u | 0x80000000)


def check_topk_own_logits(gpu_idx, gpu_w, gpu_logits, k):
    """The GPU's top-k must be exactly the first k experts of its own fp32
    logits ranked by (logit descending, expert index ascending), in that
    order, on every token; its weights within fp32 rounding of the softmax
    over those k logits.  A test-side check of the selection alone: it
    involves no oracle and needs no tolerance on the indices."""
    key = order_keys(gpu_logits)
    order = np.argsort(-key, axis=1, kind="stable")[:, :k]
    gi = np.asarray(gpu_idx)
    bad = np.nonzero((order != gi).any(axis=1))[0]
    assert bad.size == 0, ("top-k differs from the GPU's own logits at tokens",
                           bad[:10], gi[bad[:3]], order[bad[:3]])
    sel = np.take_along_axis(np.asarray(gpu_logits, dtype=np.float64), order,
                             axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    err = np.abs(np.asarray(gpu_w, dtype=np.float64) - w)
    assert err.max() <= 2e-6, ("weights vs own logits", err.max())


def check_plan_valid(topk_idx, counts, offsets, tok_row, row_src, E, pad):
    """Everything a routing plan must satisfy for the given top-k choice;
    together these fix counts, offsets, tok_row and row_src uniquely:
    counts are the per-expert histogram, offsets the exclusive scan of the
    counts rounded up to pad, expert e's tokens fill [offsets[e],
    offsets[e] + counts[e]) in ascending token order, row_src inverts
    tok_row and every other row is -1."""
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    cnt = np.bincount(idx.ravel(), minlength=E)
    assert np.array_equal(np.asarray(counts), cnt)
    seg = -(-cnt // pad) * pad
    assert np.array_equal(np.asarray(offsets, dtype=np.int64),
                          np.concatenate([[0], np.cumsum(seg)]))
    tr = np.asarray(tok_row, dtype=np.int64)
    rs = np.asarray(row_src, dtype=np.int64)
    # ascending token order inside each segment (slot order within a token
    # is irrelevant: a token picks an expert at most once)
    tok = np.repeat(np.arange(T), k)
    ex = idx.ravel()
    ordr = np.lexsort((tok, ex))
    expect = np.empty(T * k, dtype=np.int64)
    first = np.asarray(offsets, dtype=np.int64)[ex[ordr]]
    rank = np.arange(T * k) - np.concatenate([[0], np.cumsum(cnt)])[ex[ordr]]
    expect[ordr] = first + rank
    assert np.array_equal(tr.ravel(), expect), "tok_row"
    want_src = np.full(rs.shape[0], -1, dtype=np.int64)
    want_src[expect] = tok
    assert np.array_equal(rs, want_src), "row_src"
