"""Python binding of the C ABI in include/moe.h.

Argument marshalling only: every step of the transform runs in the HIP
library ``libmoe_mi355x.so``.  PyTorch provides device memory and the
current HIP stream.  There is no fallback: if the library is not built this
module raises on first use.

Low-level functions carry the C names (``moe_route``, ``moe_plan``,
``moe_dispatch``, ``moe_route_dispatch``, ``moe_route_dispatch_one_launch``,
``moe_dispatch_noalloc``,
``moe_combine_residual``, ``moe_farskip_aux``,
``moe_combine_backward``, ``moe_dispatch_backward``, ``moe_expert_gemm_fp8``,
``moe_expert_fixture``) and take preallocated tensors; ``route`` /
``route_dispatch`` / ``plan`` /
``dispatch`` / ``combine_residual`` / ``farskip_aux`` /
``combine_main_residual`` / ``combine_backward`` / ``dispatch_backward`` /
``expert_gemm_fp8`` / ``expert_fixture`` allocate their outputs with torch
and call them.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, List, Optional

import torch

from .build import LIB_PATH

MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_MAX_EXPERTS, MOE_MAX_TOPK = 512, 16
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(
    __file__))), "include", "moe.h")

_lib = None
_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t

_SIGS = {
    "moe_status_string": (ctypes.c_char_p, [_i]),
    "moe_last_hip_error": (_i, []),
    "moe_rows_capacity": (_sz, [_i, _i, _i, _i]),
    "moe_workspace_bytes": (_sz, [_i, _i, _i]),
    "moe_route": (_i, [_vp, _i, _i, _i, _vp, _i, _vp, _i, _i, _vp, _vp, _vp,
                       _vp, _vp, _vp, _sz, _vp]),
    "moe_plan": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "moe_dispatch": (_i, [_vp, _i, _i, _i, _vp, _i, _i, _i, _vp, _vp, _vp,
                          _sz, _i, _vp, _sz, _vp, _vp, _vp, _vp]),
    "moe_route_dispatch": (_i, [_vp, _i, _i, _i, _vp, _i, _vp, _i, _i, _vp,
                                _vp, _vp, _vp, _vp, _vp, _sz, _i, _vp, _sz,
                                _vp, _vp, _vp, _vp]),
    "moe_route_dispatch_one_launch": (_i, [_vp, _i, _i, _i, _vp, _i, _vp, _i,
                                           _i, _vp, _vp, _vp, _vp, _vp, _vp,
                                           _sz, _i, _vp, _sz, _vp, _vp, _vp,
                                           _vp]),
    "moe_noalloc_scratch_bytes": (_sz, [_i, _i, _i]),
    "moe_dispatch_noalloc": (_i, [_vp, _i, _i, _i, _vp, _i, _i, _i, _vp, _vp,
                                  _i, _vp, _sz, _vp, _vp, _vp, _vp]),
    "moe_combine_residual": (_i, [_vp, _i, _i, _sz, _vp, _vp, _i, _i, _vp,
                                  _vp, _vp, _vp, _vp, _i, _vp]),
    "moe_expert_fixture": (_i, [_vp, _i, _vp, _i, _vp, _vp, _i, _vp, _sz,
                                _vp, _i, _vp]),
    "moe_farskip_aux": (_i, [_vp, _vp, _vp, _i, _i, _vp]),
    "moe_expert_gemm_workspace_bytes": (_sz, [_sz, _i]),
    "moe_expert_gemm_fp8": (_i, [_vp, _vp, _i, _sz, _vp, _vp, _i, _vp, _vp,
                                 _i, _vp, _i, _vp, _sz, _vp]),
    "moe_combine_backward": (_i, [_vp, _vp, _i, _i, _sz, _vp, _vp, _i, _i,
                                  _vp, _vp, _vp]),
    "moe_dispatch_backward": (_i, [_vp, _i, _i, _sz, _vp, _i, _i, _vp, _i,
                                   _vp]),
}


def header_functions() -> List[str]:
    """Names of the functions declared in include/moe.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(moe_[a-z_]+)\s*\(", text)


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library {LIB_PATH} not built: run "
                "`python -m combine_router_gate_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().moe_status_string(status).decode()
        if status == -8:
            msg += f" (hipError {lib().moe_last_hip_error()})"
        super().__init__(f"{where}: {msg}")
        self.status = status


def _check(status: int, where: str):
    if status != 0:
        raise MoEError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.uint8:
        return MOE_FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


# ----------------------------------------------------------------- C names

def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_rows_capacity(T: int, E: int, k: int, pad: int) -> int:
    return lib().moe_rows_capacity(T, E, k, pad)


def moe_workspace_bytes(T: int, E: int, k: int) -> int:
    return lib().moe_workspace_bytes(T, E, k)


def moe_route(x, w_gate, bias, k, pad, topk_idx, topk_w, counts, offsets,
              logits_dbg, workspace, stream=None):
    T, H = x.shape
    E = w_gate.shape[0]
    st = lib().moe_route(_ptr(x), _dt(x), T, H, _ptr(w_gate), E, _ptr(bias),
                         k, pad, _ptr(topk_idx), _ptr(topk_w), _ptr(counts),
                         _ptr(offsets), _ptr(logits_dbg), _ptr(workspace),
                         workspace.numel() if workspace is not None else 0,
                         stream if stream is not None else _stream(x.device))
    _check(st, "moe_route")


def moe_plan(topk_idx, E, pad, counts, offsets, workspace, stream=None):
    T, k = topk_idx.shape
    st = lib().moe_plan(_ptr(topk_idx), T, k, E, pad, _ptr(counts),
                        _ptr(offsets), _ptr(workspace),
                        workspace.numel() if workspace is not None else 0,
                        stream if stream is not None else
                        _stream(topk_idx.device))
    _check(st, "moe_plan")


def moe_dispatch(x, topk_idx, E, pad, counts, offsets, workspace,
                 payload_dtype, rows, row_scales, row_src, tok_row,
                 stream=None):
    T, H = x.shape
    k = topk_idx.shape[1]
    st = lib().moe_dispatch(_ptr(x), _dt(x), T, H, _ptr(topk_idx), k, E, pad,
                            _ptr(counts), _ptr(offsets), _ptr(workspace),
                            workspace.numel() if workspace is not None else 0,
                            payload_dtype, _ptr(rows), rows.shape[0],
                            _ptr(row_scales), _ptr(row_src), _ptr(tok_row),
                            stream if stream is not None else
                            _stream(x.device))
    _check(st, "moe_dispatch")


def moe_route_dispatch(x, w_gate, bias, k, pad, topk_idx, topk_w, counts,
                       offsets, logits_dbg, workspace, payload_dtype, rows,
                       row_scales, row_src, tok_row, stream=None):
    T, H = x.shape
    E = w_gate.shape[0]
    st = lib().moe_route_dispatch(
        _ptr(x), _dt(x), T, H, _ptr(w_gate), E, _ptr(bias), k, pad,
        _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets),
        _ptr(logits_dbg), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, payload_dtype,
        _ptr(rows), rows.shape[0], _ptr(row_scales), _ptr(row_src),
        _ptr(tok_row), stream if stream is not None else _stream(x.device))
    _check(st, "moe_route_dispatch")


def moe_route_dispatch_one_launch(x, w_gate, bias, k, pad, topk_idx, topk_w,
                                  counts, offsets, logits_dbg, workspace,
                                  payload_dtype, rows, row_scales, row_src,
                                  tok_row, stream=None):
    T, H = x.shape
    E = w_gate.shape[0]
    st = lib().moe_route_dispatch_one_launch(
        _ptr(x), _dt(x), T, H, _ptr(w_gate), E, _ptr(bias), k, pad,
        _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets),
        _ptr(logits_dbg), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, payload_dtype,
        _ptr(rows), rows.shape[0], _ptr(row_scales), _ptr(row_src),
        _ptr(tok_row), stream if stream is not None else _stream(x.device))
    _check(st, "moe_route_dispatch_one_launch")


def moe_noalloc_scratch_bytes(T: int, E: int, k: int) -> int:
    return lib().moe_noalloc_scratch_bytes(T, E, k)


def moe_dispatch_noalloc(x, topk_idx, E, pad, counts, offsets, payload_dtype,
                         rows, row_scales, row_src, tok_row, stream=None):
    T, H = x.shape
    k = topk_idx.shape[1]
    st = lib().moe_dispatch_noalloc(
        _ptr(x), _dt(x), T, H, _ptr(topk_idx), k, E, pad, _ptr(counts),
        _ptr(offsets), payload_dtype, _ptr(rows), rows.shape[0],
        _ptr(row_scales), _ptr(row_src), _ptr(tok_row),
        stream if stream is not None else _stream(x.device))
    _check(st, "moe_dispatch_noalloc")


def moe_combine_residual(y, tok_row, topk_w, shared, residual_in,
                         residual_out, residual_no_routed, out, stream=None):
    T, k = tok_row.shape
    H = y.shape[1]
    odt = _dt(out) if out is not None else MOE_BF16
    st = lib().moe_combine_residual(
        _ptr(y), _dt(y), H, y.shape[0], _ptr(tok_row), _ptr(topk_w), T, k,
        _ptr(shared), _ptr(residual_in), _ptr(residual_out),
        _ptr(residual_no_routed), _ptr(out), odt,
        stream if stream is not None else _stream(y.device))
    _check(st, "moe_combine_residual")


def moe_expert_fixture(rows, payload_dtype, row_scales, row_src, offsets,
                       sigma, y, stream=None):
    H = y.shape[1]
    E = offsets.numel() - 1
    st = lib().moe_expert_fixture(
        _ptr(rows), payload_dtype, _ptr(row_scales), H, _ptr(row_src),
        _ptr(offsets), E, _ptr(sigma), rows.shape[0], _ptr(y), _dt(y),
        stream if stream is not None else _stream(y.device))
    _check(st, "moe_expert_fixture")


def moe_expert_gemm_workspace_bytes(rows_capacity: int, E: int) -> int:
    return lib().moe_expert_gemm_workspace_bytes(rows_capacity, E)


def moe_expert_gemm_fp8(rows, row_scales, row_src, offsets, w, w_scales, y,
                        workspace, stream=None):
    cap, K = rows.shape
    E, N = w.shape[0], w.shape[1]
    st = lib().moe_expert_gemm_fp8(
        _ptr(rows), _ptr(row_scales), K, cap, _ptr(row_src), _ptr(offsets), E,
        _ptr(w), _ptr(w_scales), N, _ptr(y), _dt(y), _ptr(workspace),
        workspace.numel() if workspace is not None else 0,
        stream if stream is not None else _stream(rows.device))
    _check(st, "moe_expert_gemm_fp8")


def moe_farskip_aux(shared, residual_in, residual_no_routed, stream=None):
    T, H = residual_in.shape
    st = lib().moe_farskip_aux(_ptr(shared), _ptr(residual_in),
                               _ptr(residual_no_routed), T, H,
                               stream if stream is not None else
                               _stream(residual_in.device))
    _check(st, "moe_farskip_aux")


def moe_combine_backward(grad_out, y, tok_row, topk_w, grad_y, grad_w,
                         stream=None):
    T, k = tok_row.shape
    H = y.shape[1]
    st = lib().moe_combine_backward(
        _ptr(grad_out), _ptr(y), _dt(y), H, y.shape[0], _ptr(tok_row),
        _ptr(topk_w), T, k, _ptr(grad_y), _ptr(grad_w),
        stream if stream is not None else _stream(y.device))
    _check(st, "moe_combine_backward")


def moe_dispatch_backward(grad_rows, tok_row, grad_x, stream=None):
    T, k = tok_row.shape
    H = grad_rows.shape[1]
    st = lib().moe_dispatch_backward(
        _ptr(grad_rows), _dt(grad_rows), H, grad_rows.shape[0], _ptr(tok_row),
        T, k, _ptr(grad_x), _dt(grad_x),
        stream if stream is not None else _stream(grad_rows.device))
    _check(st, "moe_dispatch_backward")


# ----------------------------------------------------------------- allocating

def route(x: torch.Tensor, w_gate: torch.Tensor, k: int, pad: int,
          bias: Optional[torch.Tensor] = None,
          want_logits: bool = False) -> Dict[str, torch.Tensor]:
    """Gate + top-k + histogram + scan.  Returns the routing plan."""
    T, H = x.shape
    E = w_gate.shape[0]
    dev = x.device
    p = dict(
        topk_idx=torch.empty((T, k), dtype=torch.int32, device=dev),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
        counts=torch.empty(E, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        workspace=torch.empty(max(moe_workspace_bytes(T, E, k), 1),
                              dtype=torch.uint8, device=dev),
        logits=(torch.empty((T, E), dtype=torch.float32, device=dev)
                if want_logits else None),
    )
    moe_route(x, w_gate, bias, k, pad, p["topk_idx"], p["topk_w"],
              p["counts"], p["offsets"], p["logits"], p["workspace"])
    p.update(E=E, k=k, pad=pad, T=T)
    return p


def route_dispatch(x: torch.Tensor, w_gate: torch.Tensor, k: int, pad: int,
                   bias: Optional[torch.Tensor] = None, payload: str = "same",
                   want_logits: bool = False, one_launch: bool = False):
    """moe_route + moe_dispatch in one call (small batches skip the plan
    kernel; one_launch=True calls moe_route_dispatch_one_launch).  Returns
    (plan, dispatched) like route() and dispatch()."""
    T, H = x.shape
    E = w_gate.shape[0]
    dev = x.device
    p = dict(
        topk_idx=torch.empty((T, k), dtype=torch.int32, device=dev),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
        counts=torch.empty(E, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        workspace=torch.empty(max(moe_workspace_bytes(T, E, k), 1),
                              dtype=torch.uint8, device=dev),
        logits=(torch.empty((T, E), dtype=torch.float32, device=dev)
                if want_logits else None),
    )
    p.update(E=E, k=k, pad=pad, T=T)
    cap = moe_rows_capacity(T, E, k, pad)
    fp8 = payload == "fp8"
    pdt = MOE_FP8_E4M3 if fp8 else _dt(x)
    d = dict(
        rows=torch.empty((cap, H), dtype=torch.uint8 if fp8 else x.dtype,
                         device=dev),
        row_scales=(torch.empty((cap, H // 128), dtype=torch.float32,
                                device=dev) if fp8 else None),
        row_src=torch.empty(cap, dtype=torch.int32, device=dev),
        tok_row=torch.empty((T, k), dtype=torch.int32, device=dev),
        payload_dtype=pdt,
    )
    fn = moe_route_dispatch_one_launch if one_launch else moe_route_dispatch
    fn(x, w_gate, bias, k, pad, p["topk_idx"], p["topk_w"], p["counts"],
       p["offsets"], p["logits"], p["workspace"], pdt, d["rows"],
       d["row_scales"], d["row_src"], d["tok_row"])
    return p, d


def plan(topk_idx: torch.Tensor, E: int, pad: int) -> Dict[str, torch.Tensor]:
    """Histogram + scan for externally chosen experts."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    p = dict(
        topk_idx=topk_idx,
        counts=torch.empty(E, dtype=torch.int32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        workspace=torch.empty(max(moe_workspace_bytes(T, E, k), 1),
                              dtype=torch.uint8, device=dev),
    )
    moe_plan(topk_idx, E, pad, p["counts"], p["offsets"], p["workspace"])
    p.update(E=E, k=k, pad=pad, T=T)
    return p


def dispatch(x: torch.Tensor, p: Dict, payload: str = "same",
             capacity: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Scatter token rows into the expert-major buffer (payload "same" or
    "fp8")."""
    T, H = x.shape
    E, k, pad = p["E"], p["k"], p["pad"]
    cap = capacity if capacity is not None else moe_rows_capacity(T, E, k, pad)
    dev = x.device
    fp8 = payload == "fp8"
    pdt = MOE_FP8_E4M3 if fp8 else _dt(x)
    d = dict(
        rows=torch.empty((cap, H), dtype=torch.uint8 if fp8 else x.dtype,
                         device=dev),
        row_scales=(torch.empty((cap, H // 128), dtype=torch.float32,
                                device=dev) if fp8 else None),
        row_src=torch.empty(cap, dtype=torch.int32, device=dev),
        tok_row=torch.empty((T, k), dtype=torch.int32, device=dev),
        payload_dtype=pdt,
    )
    moe_dispatch(x, p["topk_idx"], E, pad, p["counts"], p["offsets"],
                 p["workspace"], pdt, d["rows"], d["row_scales"],
                 d["row_src"], d["tok_row"])
    return d


def expert_fixture(d: Dict, p: Dict, sigma: torch.Tensor,
                   y_dtype=torch.bfloat16) -> torch.Tensor:
    rows = d["rows"]
    y = torch.empty((rows.shape[0], rows.shape[1]), dtype=y_dtype,
                    device=rows.device)
    moe_expert_fixture(rows, d["payload_dtype"], d["row_scales"],
                       d["row_src"], p["offsets"], sigma, y)
    return y


def combine_residual(y: torch.Tensor, tok_row: torch.Tensor,
                     topk_w: torch.Tensor,
                     shared: Optional[torch.Tensor] = None,
                     residual: Optional[torch.Tensor] = None,
                     out_dtype=torch.bfloat16, in_place: bool = False):
    """Weighted combine (+ dual residual).  Returns (residual_out,
    residual_no_routed) with a residual, else the routed(+shared) output."""
    T = tok_row.shape[0]
    H = y.shape[1]
    if residual is not None:
        res_out = residual if in_place else torch.empty_like(residual)
        rnr = torch.empty_like(residual)
        moe_combine_residual(y, tok_row, topk_w, shared, residual, res_out,
                             rnr, None)
        return res_out, rnr
    out = torch.empty((T, H), dtype=out_dtype, device=y.device)
    moe_combine_residual(y, tok_row, topk_w, shared, None, None, None, out)
    return out


def farskip_aux(shared: Optional[torch.Tensor],
                residual: torch.Tensor) -> torch.Tensor:
    """Auxiliary stream residual + shared (bf16), before any routing."""
    rnr = torch.empty_like(residual)
    moe_farskip_aux(shared, residual, rnr)
    return rnr


def combine_main_residual(y, tok_row, topk_w, shared, residual,
                          in_place: bool = False) -> torch.Tensor:
    """Main stream residual + routed + shared only (split form)."""
    res_out = residual if in_place else torch.empty_like(residual)
    moe_combine_residual(y, tok_row, topk_w, shared, residual, res_out, None,
                         None)
    return res_out


def combine_backward(grad_out, y, tok_row, topk_w):
    """(grad_y, grad_w) of the weighted combine; grad_y rows that no slot
    references are zero here (the kernel leaves them unwritten)."""
    T, k = tok_row.shape
    grad_y = torch.zeros((y.shape[0], y.shape[1]), dtype=torch.bfloat16,
                         device=y.device)
    grad_w = torch.empty((T, k), dtype=torch.float32, device=y.device)
    moe_combine_backward(grad_out, y, tok_row, topk_w, grad_y, grad_w)
    return grad_y, grad_w


def dispatch_backward(grad_rows, tok_row, out_dtype=torch.float32):
    """grad_x[t] = sum_j grad_rows[tok_row[t, j]]."""
    T = tok_row.shape[0]
    grad_x = torch.empty((T, grad_rows.shape[1]), dtype=out_dtype,
                         device=grad_rows.device)
    moe_dispatch_backward(grad_rows, tok_row, grad_x)
    return grad_x


def expert_gemm_fp8(d: Dict[str, torch.Tensor], p: Dict[str, torch.Tensor],
                    w: torch.Tensor, w_scales: torch.Tensor,
                    y_dtype=torch.bfloat16) -> torch.Tensor:
    """Grouped fp8 GEMM over the dispatched rows: y [rows_capacity, N].
    w: [E, N, K] uint8 E4M3 codes, w_scales: [E, N/128, K/128] fp32."""
    rows = d["rows"]
    cap = rows.shape[0]
    E, N = w.shape[0], w.shape[1]
    y = torch.empty((cap, N), dtype=y_dtype, device=rows.device)
    ws = torch.empty(max(moe_expert_gemm_workspace_bytes(cap, E), 1),
                     dtype=torch.uint8, device=rows.device)
    moe_expert_gemm_fp8(rows, d["row_scales"], d["row_src"], p["offsets"], w,
                        w_scales, y, ws)
    return y
