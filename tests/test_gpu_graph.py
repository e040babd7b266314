"""The whole path (moe_route -> moe_dispatch -> moe_combine_residual) under
HIP graph capture, through the C ABI.

The library issues no memset and allocates nothing, so one layer's launches
can be captured once and replayed.  The graph is replayed several times with
eager work and synchronisations in between, and every replay must equal the
eager result bit for bit (the kernels are deterministic).  Shapes cover the
small-batch route (split gate, one-token reduction, one-workgroup plan),
the split gate with a separate histogram and scan, and the fused-histogram
prefill path with fp8 dispatch.
"""
import numpy as np
import pytest
import torch

from combine_router_gate_amd import inputs as I
from combine_router_gate_amd import moe
from _gpu_common import note, to_dev

pytestmark = pytest.mark.gpu

C = I.CONFIGS
CASES = {
    "decode": C["dsv3_decode"],
    "t700_e64": C["dsv3_decode"].with_shape(T=700, H=512, E=64, k=4, pad=16),
    "prefill_t2048_fp8": C["dsv3_prefill"].with_shape(T=2048, H=1024),
}


def _buffers(cfg, wl):
    x, w = to_dev(wl.x), to_dev(wl.w_gate)
    b = torch.from_numpy(wl.bias).cuda() if wl.bias is not None else None
    p = moe.route(x, w, cfg.k, cfg.pad, bias=b)
    d = moe.dispatch(x, p, payload="fp8" if cfg.payload == "fp8" else "same")
    # a fixed expert output (the path is route -> dispatch -> combine; the
    # stand-in expert is not part of it)
    y = moe.expert_fixture(d, p, to_dev(wl.sigma), y_dtype=torch.bfloat16)
    shared, res = to_dev(wl.shared), to_dev(wl.residual)
    out = dict(res_out=torch.empty_like(res), rnr=torch.empty_like(res))
    return x, w, b, p, d, y, shared, res, out


def _layer(cfg, x, w, b, p, d, y, shared, res, out):
    moe.moe_route(x, w, b, cfg.k, cfg.pad, p["topk_idx"], p["topk_w"],
                  p["counts"], p["offsets"], None, p["workspace"])
    moe.moe_dispatch(x, p["topk_idx"], cfg.E, cfg.pad, p["counts"],
                     p["offsets"], p["workspace"], d["payload_dtype"],
                     d["rows"], d["row_scales"], d["row_src"], d["tok_row"])
    moe.moe_combine_residual(y, d["tok_row"], p["topk_w"], shared, res,
                             out["res_out"], out["rnr"], None)


def _snapshot(p, d, out):
    names = {"topk_idx": p["topk_idx"], "topk_w": p["topk_w"],
             "counts": p["counts"], "offsets": p["offsets"],
             "tok_row": d["tok_row"], "row_src": d["row_src"],
             "res_out": out["res_out"], "rnr": out["rnr"]}
    snap = {k: v.clone() for k, v in names.items()}
    if d["row_scales"] is not None:
        snap["row_scales"] = d["row_scales"].clone()
    # rows holding a token (padding rows are not written)
    live = (d["row_src"] >= 0).nonzero().flatten()
    snap["rows"] = d["rows"][live].clone()
    return snap


def _equal(a, b):
    for k in a:
        x, y = a[k], b[k]
        if x.dtype in (torch.bfloat16, torch.float32):
            x, y = x.view(torch.int16 if x.dtype == torch.bfloat16
                          else torch.int32), y.view(
                torch.int16 if y.dtype == torch.bfloat16 else torch.int32)
        assert torch.equal(x, y), k


@pytest.mark.parametrize("name", list(CASES))
def test_layer_graph_replays_equal_eager(name):
    cfg = CASES[name]
    note(f"graph capture {name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}")
    wl = I.make_workload(cfg, 21)
    bufs = _buffers(cfg, wl)
    x, w, b, p, d, y, shared, res, out = bufs
    torch.cuda.synchronize()
    _layer(cfg, *bufs)
    torch.cuda.synchronize()
    ref = _snapshot(p, d, out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the capture stream
        _layer(cfg, *bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _layer(cfg, *bufs)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: clobber every output
        for t in (p["topk_idx"], p["counts"], p["offsets"], d["tok_row"],
                  d["row_src"]):
            t.fill_(-7)
        out["res_out"].fill_(3.0)
        out["rnr"].fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _equal(ref, _snapshot(p, d, out))
        note(f"graph {name}: replay {rep} equals eager")
