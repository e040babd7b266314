"""CPU oracle of the MoE route -> dispatch -> combine(+FarSkip dual residual)
transform.  TEST INFRASTRUCTURE ONLY.

This module is the plain, slow definition the HIP kernels are checked
against.  Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import it; the product path never does and never falls
back to it.  It shares no code, header, table or helper with the HIP path and
imports nothing from the product package: callers hand it numpy arrays of
exact float32 values (bf16 inputs are passed widened, which is exact).

Arithmetic is float64 unless a step is defined in another precision (the
fp8 scale and the quotient x/s are float32 operations by definition; outputs
are rounded once, to nearest-even, into their storage dtype).

Sources, by page and section:
  * Router: "Efficient and Portable Mixture-of-Experts Communication"
    (Perplexity), Introduction -- the router is a small linear layer giving a
    probability distribution over experts; the top-K experts are selected and
    the output is the sum of their outputs weighted by the router's
    probabilities.
  * Counts per destination expert: same page, section "Dispatch" (one warp
    counts the tokens bound for each expert).
  * Per-expert contiguous buffers and the (expert, token) bookkeeping kept for
    combine: same page, "Dispatch" and "Combine"; fixed per-expert capacity
    bounds: section "Portable Kernels".
  * Block scaling factors travelling with fp8 tokens: same page, "Dispatch";
    DeepEP news page, technical overview (FP8 dispatch).
  * Per-expert padding (``token_padding`` = 128) and ``cu_seqlens``: "MoonEP
    developer guide", core API example and core configuration parameters.
  * Dual residual update: Instella-MoE-16B-A3B-SFT article, section on where
    the dual residual streams are implemented (the four-line update).

Readings of points the pages leave open (each listed in the design notes):
renormalised top-k weights; ties broken toward the lower expert index;
the bias added to the logits before softmax; ascending token order inside an
expert's segment; padded rows carry no data; OCP E4M3FN with scale
s = fl32(amax / 448), code = RNE-saturating E4M3 of fl32(x / s), s = 1 for an
all-zero block; blocks of 128 consecutive hidden elements.
"""
from __future__ import annotations

import numpy as np

FP8_MAX = 448.0           # largest finite OCP E4M3FN magnitude
FP8_BLOCK = 128           # hidden elements per fp8 scale


# ---------------------------------------------------------------- sizing

def rows_capacity(T: int, E: int, k: int, pad: int) -> int:
    """Upper bound on the rows of the expert-major buffer: T*k slots plus at
    most pad-1 padding rows per expert (fixed, host-known capacity as in
    "Portable Kernels": every writer gets a unique row with no
    synchronisation)."""
    return T * k + E * (pad - 1)


# ---------------------------------------------------------------- rounding

def round_to_bf16(v) -> np.ndarray:
    """Round float64 values once, to nearest with ties to even, onto the bf16
    grid (8 significant bits, exponent range of float32).  Returns float64
    values that are exactly representable in bf16."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                      # v = m * 2**e, 0.5 <= |m| < 1
    ulp_exp = np.maximum(e, -125) - 8       # bf16 spacing in [2**(e-1), 2**e)
    return np.ldexp(np.round(np.ldexp(v, -ulp_exp)), ulp_exp)


def bf16_bits(v) -> np.ndarray:
    """Storage bits of values that are exactly representable in bf16."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """float64 value of bf16 storage bits."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- O1 gate

def gate_logits(x, w_gate, bias=None) -> np.ndarray:
    """Router logits l[t, e] = sum_h x[t, h] * W[e, h] (+ bias[e]) in float64.

    The router is "a small linear layer" (Perplexity page, Introduction).
    The bias, when present, is added to the logits before the softmax."""
    x64 = np.asarray(x, dtype=np.float64)
    w64 = np.asarray(w_gate, dtype=np.float64)
    logits = x64 @ w64.T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    return logits


# ---------------------------------------------------------------- O2 top-k

def select_topk(logits, k: int):
    """Softmax over all experts, top-k selection, renormalised weights.

    Experts are ranked by logit, descending; equal logits go to the lower
    expert index first (exp is strictly increasing, so this is the order of
    the exact probabilities).  The k chosen experts are listed in that order.
    Weights: p = softmax(l) over all E experts in float64, then
    w_j = p[e_j] / sum_i p[e_i] over the k chosen, rounded to float32.
    """
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    # stable sort of -l: ties keep ascending expert index
    order = np.argsort(-l, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    m = l.max(axis=1, keepdims=True)
    ex = np.exp(l - m)
    p = ex / ex.sum(axis=1, keepdims=True)
    p_sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    w = p_sel / p_sel.sum(axis=1, keepdims=True)
    return idx, w.astype(np.float32)


# ---------------------------------------------------------------- O3/O4

def expert_counts(topk_idx, E: int) -> np.ndarray:
    """counts[e] = number of (token, slot) pairs routed to expert e."""
    return np.bincount(np.asarray(topk_idx).ravel(), minlength=E).astype(
        np.int32)


def padded_offsets(counts, pad: int) -> np.ndarray:
    """Exclusive scan of the per-expert counts, each rounded up to a multiple
    of ``pad`` (MoonEP ``token_padding``): offsets[0] = 0 and
    offsets[e+1] = offsets[e] + ceil(counts[e] / pad) * pad."""
    E = len(counts)
    off = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        off[e + 1] = off[e] + ((int(counts[e]) + pad - 1) // pad) * pad
    return off.astype(np.int32)


def route(x, w_gate, bias, k: int, pad: int) -> dict:
    """O1-O4 on the oracle's own float64 logits."""
    logits = gate_logits(x, w_gate, bias)
    idx, w = select_topk(logits, k)
    counts = expert_counts(idx, logits.shape[1])
    return dict(logits=logits, topk_idx=idx, topk_w=w, counts=counts,
                offsets=padded_offsets(counts, pad))


# ---------------------------------------------------------------- O5 slots

def assign_slots(topk_idx, offsets, E: int, capacity: int):
    """Stable slot assignment.

    Expert e's segment starts at offsets[e] and holds, in ascending token
    order, every token that chose e.  tok_row[t, j] is the row that received
    slot (t, j); row_src[r] is the token held by row r, or -1 for a row that
    holds none (padding and unused capacity)."""
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    tok_row = np.full((T, k), -1, dtype=np.int32)
    row_src = np.full(capacity, -1, dtype=np.int32)
    for e in range(E):
        ts, js = np.nonzero(idx == e)        # row-major: ascending t
        rows = int(offsets[e]) + np.arange(len(ts))
        tok_row[ts, js] = rows
        row_src[rows] = ts
    return tok_row, row_src


# ---------------------------------------------------------------- O6 fp8

def e4m3_decode(codes) -> np.ndarray:
    """float64 value of OCP FP8 E4M3FN codes: 1 sign, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent field 0 is subnormal (m * 2**-9);
    S.1111.111 is NaN; there are no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    mag = np.where(ef == 0, mf * 2.0 ** -9,
                   (1.0 + mf / 8.0) * np.ldexp(1.0, ef - 7))
    mag = np.where((ef == 15) & (mf == 7), np.nan, mag)
    return s * mag


def e4m3_encode(v) -> np.ndarray:
    """OCP FP8 E4M3FN code of float32 values: round to nearest, ties to even,
    saturating to +-448; the sign of a value that rounds to zero is kept.

    The magnitude is rounded on its own binade's grid: spacing 2**(E-3) for
    |v| in [2**E, 2**(E+1)) with E >= -6, and 2**-9 below 2**-6 (subnormals).
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    _, e = np.frexp(a)                       # a in [2**(e-1), 2**e)
    ulp_exp = np.maximum(e - 1, -6) - 3
    q = np.ldexp(np.round(np.ldexp(a, -ulp_exp)), ulp_exp)
    q = np.minimum(q, FP8_MAX)
    # encode the rounded magnitude
    _, qe = np.frexp(q)
    normal = q >= 2.0 ** -6
    ef = np.where(normal, qe - 1 + 7, 0)
    mant = np.where(normal, np.ldexp(q, -(qe - 1)) * 8.0 - 8.0,
                    q * 2.0 ** 9)
    code = (ef.astype(np.int64) << 3) | mant.astype(np.int64)
    code = code | np.where(neg, 0x80, 0)
    code = np.where(np.isnan(v), 0x7F, code)
    return code.astype(np.uint8)


def quantize_row_e4m3(x_row):
    """Quantise one hidden row to fp8 with one float32 scale per block of 128
    consecutive elements: a = max |x| over the block, s = fl32(a / 448)
    (s = 1 when a = 0), code = E4M3(fl32(x / s)).  Returns (codes, scales).
    A [n, H] array is n rows, each quantised on its own."""
    x = np.asarray(x_row, dtype=np.float32)
    H = x.shape[-1]
    assert H % FP8_BLOCK == 0
    blocks = x.reshape(-1, FP8_BLOCK)
    amax = np.abs(blocks).max(axis=1)
    scales = np.where(amax > 0, amax / np.float32(FP8_MAX),
                      np.float32(1.0)).astype(np.float32)
    q = (blocks / scales[:, None]).astype(np.float32)   # float32 quotient
    return (e4m3_encode(q).reshape(x.shape),
            scales.reshape(x.shape[:-1] + (H // FP8_BLOCK,)))


# ---------------------------------------------------------------- O6 rows

def dispatch_row(x_row, payload: str):
    """Payload written for one token row: an exact copy for "f32" (float32
    values) and "bf16" (bf16 bits), or (codes, scales) for "fp8".  A [n, H]
    array gives the payloads of n rows."""
    if payload == "f32":
        return np.asarray(x_row, dtype=np.float32).copy(), None
    if payload == "bf16":
        return bf16_bits(x_row), None
    if payload == "fp8":
        return quantize_row_e4m3(x_row)
    raise ValueError(payload)


def dispatch_rows(x, row_src, payload: str, chunk: int = 0):
    """O6 for every valid row of the expert-major buffer: row r receives the
    payload of token row_src[r] (each row exactly as ``dispatch_row`` gives
    it; rows are taken ``chunk`` at a time, by default as many as keep the
    temporaries near 32K elements).  Rows with row_src = -1 are left zero
    (their content is unspecified by definition and never compared)."""
    x = np.asarray(x, dtype=np.float32)
    src = np.asarray(row_src)
    R, H = len(src), x.shape[1]
    chunk = chunk if chunk > 0 else max(1, 32768 // H)
    dt = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[payload]
    rows = np.zeros((R, H), dtype=dt)
    scales = (np.zeros((R, H // FP8_BLOCK), dtype=np.float32)
              if payload == "fp8" else None)
    valid = np.nonzero(src >= 0)[0]
    for i in range(0, len(valid), chunk):
        rr = valid[i:i + chunk]
        p, s = dispatch_row(x[src[rr]], payload)
        rows[rr] = p
        if scales is not None:
            scales[rr] = s
    return rows, scales


# ---------------------------------------------------------------- O7 fixture

def dequantize_row(row, scales, payload: str) -> np.ndarray:
    """float32 values of a dispatched row: code * scale (a float32 product)
    for fp8, the stored value otherwise."""
    if payload == "f32":
        return np.asarray(row, dtype=np.float32)
    if payload == "bf16":
        return bf16_value(row).astype(np.float32)
    q = e4m3_decode(row).astype(np.float32).reshape(-1, FP8_BLOCK)
    return (q * np.asarray(scales, dtype=np.float32)[:, None]).reshape(-1)


def expert_fixture_row(row, scales, sigma_e, payload: str, y_dtype: str):
    """Stand-in expert (not part of the transform): y = sigma_e * deq(row),
    a float32 product, stored as float32 or rounded once to bf16 (bits)."""
    y = (np.float32(sigma_e) * dequantize_row(row, scales, payload)).astype(
        np.float32)
    if y_dtype == "f32":
        return y
    return bf16_bits(round_to_bf16(y))


def expert_gemm_fp8(rows, row_scales, w_codes, w_scales, e: int):
    """fp8 grouped GEMM of expert e over the given rows of its segment
    (the expert GEMM between dispatch and combine: Perplexity page,
    Dispatch; FP8 tokens with block scaling factors: DeepEP news, technical
    overview).  Each 128-wide block b contributes its exact sum of decoded
    products times the block's two scales:
      y[r, n] = sum_b sa[r, b] * sw[e, n // 128, b]
                * sum_{h in b} E4M3(rows[r, h]) * E4M3(w[e, n, h])
    rows: [m, K] codes, row_scales: [m, K/128]; float64 result [m, N]."""
    a = e4m3_decode(rows)
    wd = e4m3_decode(w_codes[e])
    sa = np.asarray(row_scales, dtype=np.float64)
    sw = np.asarray(w_scales[e], dtype=np.float64)
    m, K = a.shape
    N = wd.shape[0]
    y = np.zeros((m, N), dtype=np.float64)
    for b in range(K // 128):
        part = a[:, 128 * b:128 * (b + 1)] @ wd[:, 128 * b:128 * (b + 1)].T
        y += sa[:, b:b + 1] * part * np.repeat(sw[:, b], 128)[None, :]
    return y


def expert_of_row(offsets, r: int) -> int:
    """Expert whose padded segment [offsets[e], offsets[e+1]) holds row r."""
    return int(np.searchsorted(np.asarray(offsets), r, side="right") - 1)


# ---------------------------------------------------------------- O8/O9

def combine_token(y_rows, w) -> np.ndarray:
    """Weighted gather-combine for one token, float64:
    routed = sum_j w[j] * y_j (Perplexity page, Introduction and "Combine":
    the weighted average of the selected experts' outputs)."""
    y = np.asarray(y_rows, dtype=np.float64)
    acc = np.zeros(y.shape[-1], dtype=np.float64)
    for j in range(y.shape[0]):
        acc += np.float64(w[j]) * y[j]
    return acc


def combine(y_values, tok_row, topk_w) -> np.ndarray:
    """O8 for every token: routed[t] = sum_j w[t, j] * y[tok_row[t, j]]."""
    y = np.asarray(y_values, dtype=np.float64)
    T, k = np.asarray(tok_row).shape
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(k):
        out += np.asarray(topk_w[:, j], dtype=np.float64)[:, None] * \
            y[np.asarray(tok_row[:, j], dtype=np.int64)]
    return out


def farskip_update(routed64, shared, residual):
    """FarSkip-Collective dual residual update (Instella-MoE article, the
    four-line update): the MoE output is routed + shared;
    residual_no_routed = residual + shared and residual = residual + MoE
    output.  Sums in float64, each output rounded once to bf16.

    Returns (residual_out, residual_no_routed, residual_out_exact) where the
    first two are bf16 bits and the last is the float64 value before
    rounding."""
    r = np.asarray(residual, dtype=np.float64)
    s = np.zeros_like(r) if shared is None else np.asarray(shared,
                                                          dtype=np.float64)
    mlp_output = np.asarray(routed64, dtype=np.float64) + s
    res_exact = r + mlp_output
    rnr = r + s
    return (bf16_bits(round_to_bf16(res_exact)),
            bf16_bits(round_to_bf16(rnr)), res_exact)


def combine_backward(grad_out, y_values, tok_row, topk_w, y_rows: int):
    """Gradient of the weighted combine routed[t] = sum_j w[t, j] *
    y[tok_row[t, j]] for an upstream gradient grad_out = dL/d routed.  The
    backward pass runs through the forward routing plan ("MoonEP developer
    guide", core API example, backward); the gradients themselves are the
    chain rule of a bilinear map:
      dL/dy[tok_row[t, j]] = w[t, j] * grad_out[t]
      dL/dw[t, j]          = <grad_out[t], y[tok_row[t, j]]>
    Float64.  Returns (grad_y [y_rows, H], grad_w [T, k]); rows of grad_y that
    no slot references are zero."""
    g = np.asarray(grad_out, dtype=np.float64)
    y = np.asarray(y_values, dtype=np.float64)
    tr = np.asarray(tok_row, dtype=np.int64)
    T, k = tr.shape
    grad_y = np.zeros((y_rows, g.shape[1]), dtype=np.float64)
    grad_w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            r = tr[t, j]
            grad_y[r] = np.float64(topk_w[t, j]) * g[t]
            grad_w[t, j] = np.dot(g[t], y[r])
    return grad_y, grad_w


def dispatch_backward(grad_rows, tok_row) -> np.ndarray:
    """Gradient of the scatter: every row of the expert-major buffer holds a
    copy of its token, so dL/dx[t] = sum_j dL/drows[tok_row[t, j]] (float64;
    the transpose of the row copy of the dispatch step)."""
    gr = np.asarray(grad_rows, dtype=np.float64)
    tr = np.asarray(tok_row, dtype=np.int64)
    T, k = tr.shape
    out = np.zeros((T, gr.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            out[t] += gr[tr[t, j]]
    return out


def routed_output(routed64, out_dtype: str):
    """Routed-only output (no residual): float32 values or bf16 bits."""
    if out_dtype == "f32":
        return np.asarray(routed64, dtype=np.float64).astype(np.float32)
    return bf16_bits(round_to_bf16(routed64))
