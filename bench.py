"""Benchmark of the MoE route -> dispatch -> combine(+dual residual) layer
transform on one MI355X.

One step = moe_route (gate GEMM, top-k, histogram, scan) + moe_dispatch
(stable scatter, fp8 1x128 quantisation on the DeepSeek-V3 prefill shape) +
moe_combine_residual (weighted gather + FarSkip dual residual), on inputs
already resident in HBM.  The stand-in expert between dispatch and combine is
not part of the transform: its output is produced once before timing (the
dispatched rows, and hence the expert output, are identical every step).

Prints one JSON line.  ms_per_step: K steps launched back to back between
two events.  value = achieved HBM GB/s of dispatch + combine (algorithmic
bytes / their time, from K further steps with an event between stages), the
headline metric; the line also carries per-stage times, the roofline of the
dominant kernel (combine), the CPU-oracle baseline and, unless --no-extras,
the fp8 expert GEMM, the backward passes, the FarSkip split/overlap and a
HIP-graph replay of the layer.
"""
import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E peak, GB/s
# Kernel sources whose hash keys the committed counter-based traffic figure
COMBINE_SOURCES = ["combine_router_gate_amd/csrc/combine.hip",
                   "combine_router_gate_amd/csrc/moe_device.h"]
TRAFFIC_PROFILE = "profiles/traffic_combine_kernel_dsv3_prefill.txt"


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(workload):
    """HBM bytes per combine launch measured with FETCH_SIZE/WRITE_SIZE
    (scaled by a plain copy of known size), or None when no summary exists
    for this workload or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                key, val = ln.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("workload") != workload:
        return None
    if kv.get("sources_sha256") != sources_sha256(COMBINE_SOURCES):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None
METRIC = ("dispatch+combine µs/layer and achieved HBM GB/s (% of peak), "
          "DSV3 shape")


def algorithmic_bytes(cfg):
    """Bytes each stage must move at minimum (padding rows excluded):
    route    x once, gate weight once, top-k ids + weights written, counts
             and offsets
    dispatch x once, k payload copies (+ fp8 scales), topk_idx read,
             tok_row and row_src written
    combine  k expert rows per token, tok_row + weights, then residual and
             shared read and two bf16 streams written (or one routed output)
    """
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    S = T * k
    bx = 4 if cfg.x_dtype == "f32" else 2
    bq = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.payload]
    by = 4 if cfg.y_dtype == "f32" else 2
    route = T * H * bx + E * H * bx + S * 8 + 8 * E
    dispatch = T * H * bx + S * H * bq + 3 * S * 4
    if cfg.payload == "fp8":
        dispatch += S * (H // 128) * 4
    combine = S * H * by + S * 8
    if cfg.residual:
        combine += 4 * T * H * 2
    else:
        combine += T * H * by
    return dict(route=route, dispatch=dispatch, combine=combine)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _shared_array(shape, dtype):
    """Zeroed array in anonymous shared memory: workers forked after its
    creation write into the same pages the parent reads."""
    import mmap
    n = int(np.prod(shape)) * np.dtype(dtype).itemsize
    buf = mmap.mmap(-1, max(n, 1))
    return np.frombuffer(buf, dtype=dtype, count=int(np.prod(shape))).reshape(
        shape)


# Inputs and outputs of the CPU-baseline stages, set before the worker pool
# is forked so that the workers inherit them.
_CPU = {}


def _cpu_route(span):
    from oracle import moe_oracle as O
    c = _CPU
    lo, hi = span
    logits = O.gate_logits(c["x"][lo:hi], c["w"], c["bias"])
    idx, w = O.select_topk(logits, c["k"])
    c["idx"][lo:hi] = idx
    c["tw"][lo:hi] = w


def _cpu_dispatch(span):
    from oracle import moe_oracle as O
    c = _CPU
    lo, hi = span
    rows, scales = O.dispatch_rows(c["x"], c["row_src"][lo:hi], c["payload"])
    c["rows"][lo:hi] = rows
    if scales is not None:
        c["scales"][lo:hi] = scales


def _cpu_fixture(span):
    from oracle import moe_oracle as O
    c = _CPU
    lo, hi = span
    for r in range(lo, hi):
        if c["row_src"][r] < 0:
            continue
        e = O.expert_of_row(c["offsets"], r)
        yv = O.expert_fixture_row(c["rows"][r], None if c["scales"] is None
                                  else c["scales"][r], c["sigma"][e],
                                  c["payload"], c["y_dtype"])
        c["y"][r] = yv if c["y_dtype"] == "f32" else O.bf16_value(yv)


def _cpu_combine(span):
    from oracle import moe_oracle as O
    c = _CPU
    lo, hi = span
    k, H = c["k"], c["y"].shape[1]
    g = max(1, 65536 // (k * H))      # tokens per call: cache-sized arrays
    for a in range(lo, hi, g):
        b = min(hi, a + g)
        tr = c["tok_row"][a:b]
        n = b - a
        routed = O.combine(c["y"][tr.ravel()], np.arange(n * k).reshape(n, k),
                           c["tw"][a:b])
        if c["residual"] is not None:
            res, rnr, _ = O.farskip_update(routed, c["shared"][a:b],
                                           c["residual"][a:b])
            c["out"][a:b] = res
            c["rnr"][a:b] = rnr
        else:
            c["out"][a:b] = O.routed_output(routed, c["y_dtype"]).view(
                c["out"].dtype)


def _spans(n, parts):
    step = max(1, -(-n // parts))
    return [(a, min(n, a + step)) for a in range(0, n, step)]


def cpu_baseline(cfg, wl, n_tokens, workers):
    """The oracle on the first n_tokens tokens of the same workload (same H,
    E, k, pad, payload, expert and residual), timed twice on the host cores:
    one thread, then split over ``workers`` forked processes (tokens for the
    route and combine, rows for the dispatch; each worker single-threaded).
    Both runs call the same oracle functions on chunks of tokens or rows;
    every token and row is computed on its own, so the results are the
    same.  Must run before the GPU is initialised (the workers are
    forked)."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    from oracle import moe_oracle as O

    sub = cfg.with_shape(T=n_tokens)
    T, H, E, k, pad = sub.T, sub.H, sub.E, sub.k, sub.pad
    cap = O.rows_capacity(T, E, k, pad)
    pdt = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[sub.payload]
    c = _CPU
    c.clear()
    c.update(x=wl.x.values[:T], w=wl.w_gate.values, bias=wl.bias, k=k,
             payload=sub.payload, y_dtype=sub.y_dtype, sigma=wl.sigma,
             shared=(wl.shared.values[:T] if wl.shared is not None else None),
             residual=(wl.residual.values[:T] if wl.residual is not None
                       else None))
    c["idx"] = _shared_array((T, k), np.int32)
    c["tw"] = _shared_array((T, k), np.float32)
    c["rows"] = _shared_array((cap, H), pdt)
    c["scales"] = (_shared_array((cap, H // 128), np.float32)
                   if sub.payload == "fp8" else None)
    c["y"] = _shared_array((cap, H), np.float32)
    c["out"] = _shared_array((T, H), np.float32 if (
        sub.y_dtype == "f32" and not sub.residual) else np.uint16)
    c["rnr"] = _shared_array((T, H), np.uint16)
    c["tok_row"] = _shared_array((T, k), np.int32)
    c["row_src"] = _shared_array((cap,), np.int32)
    c["offsets"] = _shared_array((E + 1,), np.int32)

    def run(pool, n_chunks):
        go = (lambda f, spans: pool.map(f, spans)) if pool is not None else \
            (lambda f, spans: [f(sp) for sp in spans])
        t0 = time.perf_counter()
        go(_cpu_route, _spans(T, n_chunks))
        counts = O.expert_counts(c["idx"], E)
        offsets = O.padded_offsets(counts, pad)
        t1 = time.perf_counter()
        tok_row, row_src = O.assign_slots(c["idx"], offsets, E, cap)
        c["tok_row"][:] = tok_row
        c["row_src"][:] = row_src
        c["offsets"][:] = offsets
        go(_cpu_dispatch, _spans(cap, n_chunks))
        t2 = time.perf_counter()
        go(_cpu_fixture, _spans(cap, n_chunks))         # stand-in expert
        t3 = time.perf_counter()
        go(_cpu_combine, _spans(T, n_chunks))
        t4 = time.perf_counter()
        return t1 - t0, t2 - t1, t4 - t3

    b = algorithmic_bytes(sub)
    with threadpool_limits(limits=1):
        print(f"cpu baseline: one thread, {T} tokens", file=sys.stderr,
              flush=True)
        one = run(None, 16)
        first = {key: c[key].copy() for key in ("idx", "out", "rnr")}
        print(f"cpu baseline: {workers} processes", file=sys.stderr,
              flush=True)
        ctx = mp.get_context("fork")
        with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
            allc = run(pool, 4 * workers)
    for key, v in first.items():      # the two runs computed the same
        assert np.array_equal(c[key], v), key
    c.clear()

    def rate(t):
        return round((b["dispatch"] + b["combine"]) / (t[1] + t[2]) / 1e9, 4)
    return {
        "value": rate(allc), "unit": "GB/s", "cores": workers,
        "kind": "oracle",
        "sample": (f"first {n_tokens} of {cfg.T} tokens of the {cfg.name} "
                   f"workload (H={cfg.H}, E={cfg.E}, k={cfg.k}, pad={cfg.pad}, "
                   f"payload={cfg.payload}); numpy fp64 oracle split over "
                   f"{workers} single-threaded processes (dispatch + combine "
                   f"bytes over their time; route and the stand-in expert "
                   f"timed apart)"),
        "cpu_model": _cpu_model(),
        "route_s": round(allc[0], 3), "dispatch_s": round(allc[1], 3),
        "combine_s": round(allc[2], 3),
        "single_thread": {"value": rate(one), "unit": "GB/s", "cores": 1,
                          "route_s": round(one[0], 3),
                          "dispatch_s": round(one[1], 3),
                          "combine_s": round(one[2], 3)},
    }


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _mean_ms(pairs):
    return float(np.mean([a.elapsed_time(b) for a, b in pairs]))


def measure_cold(step, stream, dev, iters=10, flush_mb=1024):
    """Per-stage times with the caches (L2 and the 256 MB MALL) flushed
    before every iteration by writing flush_mb MiB of scratch."""
    import torch
    flush = torch.empty(flush_mb << 20, dtype=torch.uint8, device=dev)
    evs = []
    for i in range(iters):
        flush.fill_(i & 0xFF)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        step(ev)
        evs.append(ev)
    torch.cuda.synchronize()
    del flush
    return {
        "route_us": round(_mean_ms([(e[0], e[1]) for e in evs]) * 1e3, 2),
        "dispatch_us": round(_mean_ms([(e[1], e[2]) for e in evs]) * 1e3, 2),
        "combine_us": round(_mean_ms([(e[2], e[3]) for e in evs]) * 1e3, 2),
        "iters": iters, "flush_mib": flush_mb,
    }


def measure_copy(stream, dev, mib=1024, iters=10):
    """A plain device-to-device copy of mib MiB (torch copy_, on the launch
    stream) timed in the same session: the bandwidth an HBM-bound kernel on
    this box can be held against besides the nominal peak."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(iters):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / iters
    del src, dst
    return {"gbs": round(2 * n / (us * 1e-6) / 1e9, 1), "us": round(us, 2),
            "bytes_moved": 2 * n,
            "how": f"torch copy_ of {mib} MiB device to device, mean of "
                   f"{iters}"}


def measure_backward(cfg, moe, y, tok_row, topk_w, stream, dev, iters=10):
    """moe_combine_backward and moe_dispatch_backward through the forward
    plan: times and achieved GB/s on their algorithmic bytes."""
    import torch
    T, H, k = cfg.T, cfg.H, cfg.k
    S = T * k
    by = 4 if cfg.y_dtype == "f32" else 2
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    g = torch.randn((T, H), generator=gen, device=dev).to(torch.bfloat16)
    grad_y = torch.zeros((y.shape[0], H), dtype=torch.bfloat16, device=dev)
    grad_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    grad_x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    sp = stream.cuda_stream

    def once(ev=None):
        if ev:
            ev[0].record(stream)
        moe.moe_combine_backward(g, y, tok_row, topk_w, grad_y, grad_w, sp)
        if ev:
            ev[1].record(stream)
        moe.moe_dispatch_backward(grad_y, tok_row, grad_x, sp)
        if ev:
            ev[2].record(stream)
    once()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
           for _ in range(iters)]
    for ev in evs:
        once(ev)
    torch.cuda.synchronize()
    cb_us = _mean_ms([(e[0], e[1]) for e in evs]) * 1e3
    db_us = _mean_ms([(e[1], e[2]) for e in evs]) * 1e3
    cb_bytes = T * H * 2 + S * H * by + S * H * 2 + S * 8 + S * 4
    db_bytes = S * H * 2 + T * H * 2 + S * 4
    return {
        "combine_backward_us": round(cb_us, 2),
        "combine_backward_gbs": round(cb_bytes / (cb_us * 1e-6) / 1e9, 1),
        "dispatch_backward_us": round(db_us, 2),
        "dispatch_backward_gbs": round(db_bytes / (db_us * 1e-6) / 1e9, 1),
        "bytes": {"combine_backward": cb_bytes, "dispatch_backward": db_bytes},
        "grad_dtype": "bf16",
    }


PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA peak, TFLOP/s


def measure_expert_gemm(cfg, moe, d, p, dev, iters=5):
    """The fp8 grouped expert GEMM (moe_expert_gemm_fp8) on the dispatched
    fp8 buffer: every expert maps H -> H with synthetic E4M3 weights and
    128x128 block scales generated on the device.  FLOPs count the T*k
    routed rows (the padded rows the kernel also computes are reported
    separately)."""
    import torch
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    N = K = H
    gen = torch.Generator(device=dev)
    gen.manual_seed(13)
    w = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
    for e in range(E):
        # exponent field <= 7 (magnitudes <= 1.875): no NaN codes
        w[e] = torch.randint(0, 256, (N, K), generator=gen, device=dev,
                             dtype=torch.uint8) & 0xBF
    w_scales = (torch.rand((E, N // 128, K // 128), generator=gen,
                           device=dev) + 0.5) / float(np.sqrt(K))
    cap = d["rows"].shape[0]
    y = torch.empty((cap, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(moe.moe_expert_gemm_workspace_bytes(cap, E),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def once():
        moe.moe_expert_gemm_fp8(d["rows"], d["row_scales"], d["row_src"],
                                p["offsets"], w, w_scales, y, ws,
                                stream.cuda_stream)
    once()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(iters):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        once()
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    us = _mean_ms(pairs) * 1e3
    R = int(p["offsets"][-1].item())
    flop = 2.0 * T * k * N * K
    tf = flop / (us * 1e-6) / 1e12
    del w, y
    return {
        "us": round(us, 1), "tflops": round(tf, 1),
        "tflops_padded_rows": round(2.0 * R * N * K / (us * 1e-6) / 1e12, 1),
        "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
        "shape": f"{E} experts x [{R} padded rows ({T * k} routed), K={K}] "
                 f"x [K, N={N}] fp8 -> bf16",
    }


def measure_route_dispatch(cfg, moe, x, w, bias, p, d, y, combine, stream,
                           iters=20, reps=7):
    """Small batches: moe_route_dispatch (route + scatter, no plan kernel)
    against moe_route followed by moe_dispatch and (bf16, up to 256 tokens
    and 512 experts) against moe_route_dispatch_one_launch, alone and as a
    whole layer step with the combine; each timed over iters back-to-back
    launches."""
    import torch
    T, E, k, pad = cfg.T, cfg.E, cfg.k, cfg.pad
    sp = stream.cuda_stream

    def fused():
        moe.moe_route_dispatch(x, w, bias, k, pad, p["topk_idx"],
                               p["topk_w"], p["counts"], p["offsets"], None,
                               p["workspace"], d["payload_dtype"], d["rows"],
                               d["row_scales"], d["row_src"], d["tok_row"],
                               sp)

    def one_launch():
        moe.moe_route_dispatch_one_launch(
            x, w, bias, k, pad, p["topk_idx"], p["topk_w"], p["counts"],
            p["offsets"], None, p["workspace"], d["payload_dtype"], d["rows"],
            d["row_scales"], d["row_src"], d["tok_row"], sp)

    def separate():
        moe.moe_route(x, w, bias, k, pad, p["topk_idx"], p["topk_w"],
                      p["counts"], p["offsets"], None, p["workspace"], sp)
        moe.moe_dispatch(x, p["topk_idx"], E, pad, p["counts"], p["offsets"],
                         p["workspace"], d["payload_dtype"], d["rows"],
                         d["row_scales"], d["row_src"], d["tok_row"], sp)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(iters):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / iters

    legs = {"fused_us": fused, "separate_us": separate,
            "fused_step_us": lambda: (fused(), combine()),
            "separate_step_us": lambda: (separate(), combine())}
    one = (T <= 256 and E <= 512 and x.dtype == torch.bfloat16)
    if one:
        legs["one_launch_us"] = one_launch
        legs["one_launch_step_us"] = lambda: (one_launch(), combine())
    # the legs alternate, reps rounds, and each reports its median: these
    # launch-bound timings drift with the clock over a run
    samples = {kk: [] for kk in legs}
    for _ in range(reps):
        for kk, fn in legs.items():
            samples[kk].append(timed(fn))
    r = {kk: round(statistics.median(v), 2) for kk, v in samples.items()}
    r["how"] = (f"{iters} back-to-back calls: route+dispatch in one call "
                "(plan rebuilt in every scatter workgroup) vs moe_route then "
                "moe_dispatch"
                + (" vs moe_route_dispatch_one_launch (one kernel, two "
                   "grid-wide waits)" if one else "")
                + f"; step = with the combine; median of {reps} alternating "
                "rounds")
    return r


def measure_graph(layer, stream, iters=20):
    """One layer (route + dispatch + combine) captured once into a HIP graph
    and replayed: µs per replay, against the same launches issued eagerly.
    The path issues no memset and allocates nothing, so it captures as is."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        layer()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    torch.cuda.synchronize()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(iters):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / iters
    return {"graph_us_per_layer": round(timed(g.replay), 2),
            "eager_us_per_layer": round(timed(layer), 2), "replays": iters}


def measure_farskip_overlap(cfg, moe, y, tok_row, topk_w, shared, resid,
                            stream, dev, iters=10, n_next=2112):
    """FarSkip split form on one GPU: the auxiliary residual stream first
    (moe_farskip_aux), then the routed combine into the main stream on one
    stream while a stand-in next-layer attention projection
    (residual_no_routed @ W, [T, H] x [H, n_next] bf16, torch.matmul) runs on
    a second stream of the same priority.  Reports each part alone, the two
    in sequence and overlapped, and the combine time hidden."""
    import torch
    T, H = cfg.T, cfg.H
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    wq = (torch.randn((H, n_next), generator=gen, device=dev) /
          float(np.sqrt(H))).to(torch.bfloat16)
    rnr = torch.empty_like(resid)
    res_out = torch.empty_like(resid)
    q = torch.empty((T, n_next), dtype=torch.bfloat16, device=dev)
    s2 = torch.cuda.Stream(device=dev)
    sp = stream.cuda_stream

    def aux():
        moe.moe_farskip_aux(shared, resid, rnr, sp)

    def main_combine():
        moe.moe_combine_residual(y, tok_row, topk_w, shared, resid, res_out,
                                 None, None, sp)

    def gemm():
        torch.matmul(rnr, wq, out=q)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        pairs = []
        for _ in range(iters):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            pairs.append((a, b))
        torch.cuda.synchronize()
        return _mean_ms(pairs) * 1e3

    def sequential():
        aux()
        main_combine()
        gemm()

    def overlapped():
        aux()
        ready = torch.cuda.Event()
        ready.record(stream)
        s2.wait_event(ready)
        with torch.cuda.stream(s2):
            gemm()
        main_combine()
        stream.wait_stream(s2)

    t_aux, t_comb, t_gemm = timed(aux), timed(main_combine), timed(gemm)
    t_seq, t_ovl = timed(sequential), timed(overlapped)
    return {
        "aux_us": round(t_aux, 2), "combine_main_us": round(t_comb, 2),
        "next_gemm_us": round(t_gemm, 2),
        "next_gemm": f"[{T},{H}] x [{H},{n_next}] bf16 (torch.matmul)",
        "sequential_us": round(t_seq, 2), "overlapped_us": round(t_ovl, 2),
        "hidden_us": round(t_seq - t_ovl, 2),
        "hidden_frac_of_combine": round((t_seq - t_ovl) / t_comb, 3),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="dsv3_prefill")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-tokens", type=int, default=16384,
                    help="tokens in the CPU-oracle baseline sample, at most "
                    "the workload's (0 = skip)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the backward and FarSkip-overlap measurements "
                    "that follow the timed steps")
    ap.add_argument("--no-cold-cache", action="store_true",
                    help="skip the stage times with L2 and MALL flushed "
                    "before every iteration")
    ap.add_argument("--workers", type=int,
                    default=min(16, len(os.sched_getaffinity(0))),
                    help="host processes of the all-cores CPU-oracle run")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="run one plain device-to-device copy of this many "
                    "MiB before timing (reference for byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures the single-GPU transform only; there is "
              "no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    from combine_router_gate_amd import inputs as I

    cfg = I.CONFIGS[args.config]
    wl = I.make_workload(cfg, args.seed)
    # the CPU-oracle baseline first: its worker processes are forked, which
    # must happen before this process initialises the GPU
    cpu = None
    if args.cpu_tokens > 0:
        cpu = cpu_baseline(cfg, wl, min(args.cpu_tokens, cfg.T), args.workers)

    import torch
    from combine_router_gate_amd import moe
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(t):
        if t.dtype == "f32":
            return torch.from_numpy(t.bits).to(dev)
        return torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16).to(dev)

    T, H, E, k, pad = cfg.T, cfg.H, cfg.E, cfg.k, cfg.pad
    x, w = to_dev(wl.x), to_dev(wl.w_gate)
    bias = torch.from_numpy(wl.bias).to(dev) if wl.bias is not None else None
    shared = to_dev(wl.shared) if wl.shared is not None else None
    resid = to_dev(wl.residual) if wl.residual is not None else None
    sigma = torch.from_numpy(wl.sigma).to(dev)

    # buffers allocated once and reused by every step
    p = moe.route(x, w, k, pad, bias=bias)
    d = moe.dispatch(x, p, payload="fp8" if cfg.payload == "fp8" else "same")
    y = moe.expert_fixture(d, p, sigma,
                           y_dtype=torch.float32 if cfg.y_dtype == "f32"
                           else torch.bfloat16)
    if resid is not None:
        res_out, rnr = torch.empty_like(resid), torch.empty_like(resid)
        out = None
    else:
        res_out = rnr = None
        out = torch.empty((T, H), dtype=y.dtype, device=dev)
    torch.cuda.synchronize()

    if args.copy_calibration_mb > 0:
        nbytes = args.copy_calibration_mb << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        moe.moe_route(x, w, bias, k, pad, p["topk_idx"], p["topk_w"],
                      p["counts"], p["offsets"], None, p["workspace"], sp)
        if ev is not None:
            ev[1].record(stream)
        moe.moe_dispatch(x, p["topk_idx"], E, pad, p["counts"], p["offsets"],
                         p["workspace"], d["payload_dtype"], d["rows"],
                         d["row_scales"], d["row_src"], d["tok_row"], sp)
        if ev is not None:
            ev[2].record(stream)
        moe.moe_combine_residual(y, d["tok_row"], p["topk_w"], shared, resid,
                                 res_out, rnr, out, sp)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: K steps launched back to back
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    # stage breakdown: K more steps with an event between stages (events
    # between launches add a little time to the smallest workloads, so they
    # stay out of the timed region above)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
           for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    r_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    d_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    c_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])

    b = algorithmic_bytes(cfg)
    dc_us = (d_ms.mean() + c_ms.mean()) * 1e3
    dc_gbs = (b["dispatch"] + b["combine"]) / (dc_us * 1e-6) / 1e9
    comb_gbs = b["combine"] / (c_ms.mean() * 1e-3) / 1e9
    disp_gbs = b["dispatch"] / (d_ms.mean() * 1e-3) / 1e9
    route_gflop = 2.0 * T * H * E / 1e9

    line = {
        "metric": METRIC,
        "value": round(dc_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "H": H, "E": E, "k": k,
                   "pad": pad, "x": cfg.x_dtype,
                   "payload": "fp8_e4m3_1x128" if cfg.payload == "fp8"
                   else cfg.payload,
                   "expert_out": cfg.y_dtype,
                   "combine": "fp32 acc -> bf16, FarSkip dual residual"
                   if cfg.residual else "fp32 acc, routed only",
                   "seed": args.seed},
        "dc_us_per_layer": round(dc_us, 2),
        "dc_pct_of_peak": round(100.0 * dc_gbs / PEAK_HBM_GBS, 1),
        "route_us": round(r_ms.mean() * 1e3, 2),
        "dispatch_us": round(d_ms.mean() * 1e3, 2),
        "combine_us": round(c_ms.mean() * 1e3, 2),
        "dispatch_gbs": round(disp_gbs, 1),
        "route_tflops": round(route_gflop / (r_ms.mean() * 1e-3) / 1e3, 2),
        "bytes": b,
        "roofline": {
            "kernel": "combine_kernel (moe_combine_residual)",
            "bound": "hbm",
            "achieved": round(comb_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(comb_gbs / PEAK_HBM_GBS, 4),
            "traffic": profiled_traffic(cfg.name),
            "traffic_unit": "bytes per launch (HBM read + write)",
        },
    }
    dc = (d_ms + c_ms) * 1e3
    line["dc_us_p10_p50_p90"] = [round(float(np.percentile(dc, q)), 2)
                                 for q in (10, 50, 90)]
    copy = measure_copy(stream, dev)
    line["copy_bw"] = copy
    line["dc_frac_of_copy"] = round(dc_gbs / copy["gbs"], 4)
    if not args.no_cold_cache:
        cold = measure_cold(step, stream, dev)
        cdc = cold["dispatch_us"] + cold["combine_us"]
        cgbs = (b["dispatch"] + b["combine"]) / (cdc * 1e-6) / 1e9
        cold.update(dc_us=round(cdc, 2), dc_gbs=round(cgbs, 1),
                    dc_pct_of_peak=round(100.0 * cgbs / PEAK_HBM_GBS, 1))
        line["cold_cache"] = cold
    if not args.no_extras and T <= 512:
        line["route_dispatch"] = measure_route_dispatch(
            cfg, moe, x, w, bias, p, d, y,
            lambda: moe.moe_combine_residual(y, d["tok_row"], p["topk_w"],
                                             shared, resid, res_out, rnr,
                                             out, sp), stream)
    if not args.no_extras:
        def layer():   # the timed step's launches, on the current stream
            moe.moe_route(x, w, bias, k, pad, p["topk_idx"], p["topk_w"],
                          p["counts"], p["offsets"], None, p["workspace"])
            moe.moe_dispatch(x, p["topk_idx"], E, pad, p["counts"],
                             p["offsets"], p["workspace"], d["payload_dtype"],
                             d["rows"], d["row_scales"], d["row_src"],
                             d["tok_row"])
            moe.moe_combine_residual(y, d["tok_row"], p["topk_w"], shared,
                                     resid, res_out, rnr, out)
        line["hip_graph"] = measure_graph(layer, stream)
    if not args.no_extras and cfg.payload == "fp8":
        line["expert_gemm"] = measure_expert_gemm(cfg, moe, d, p, dev)
    if not args.no_extras:
        line["backward"] = measure_backward(cfg, moe, y, d["tok_row"],
                                            p["topk_w"], stream, dev)
        if resid is not None:
            line["farskip_overlap"] = measure_farskip_overlap(
                cfg, moe, y, d["tok_row"], p["topk_w"], shared, resid,
                stream, dev)
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
