// C ABI of the MoE route / dispatch / combine library (declared in
// include/moe.h): host-side argument validation, then kernel launches on the
// caller's stream.  Nothing here allocates, frees or synchronises.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "expert_gemm.h"
#include "moe_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

struct Span {
  const void* p;
  size_t bytes;
};

bool overlap(Span a, Span b) {
  if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0)
    return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool any_overlap(const Span* outs, int n_out, const Span* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

bool aligned(const void* p, size_t a) {
  return p == nullptr || ((uintptr_t)p % a) == 0;
}

size_t dtype_size(int dt) {
  return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : dt == MOE_FP8_E4M3 ? 1 : 0;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = (int)e;
  return MOE_ERR_HIP;
}

bool trace_on() {
  static const bool on = [] {
    const char* v = std::getenv("MOE_TRACE");
    return v != nullptr && v[0] != '\0' && v[0] != '0';
  }();
  return on;
}

// Router shape limits shared by route / plan / dispatch.
int check_route_shape(int T, int E, int k, int pad) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK ||
      k > E || pad < 1)
    return MOE_ERR_SHAPE;
  // every row index must fit in int32
  const long long cap = (long long)T * k + (long long)E * (pad - 1);
  if (cap > 0x7fffffffLL - pad) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// A gate over more than moe::kGateWideE experts takes bf16 x and at most
// moe::kSplitMaxT tokens.
int check_gate_wide(int T, int E, int x_dtype) {
  if (E <= moe::kGateWideE) return MOE_OK;
  if (x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (T > moe::kSplitMaxT) return MOE_ERR_SHAPE;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: size out of range or inconsistent";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE: unsupported dtype or dtype combination";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: pointer not aligned (16 bytes for vector arrays)";
    case MOE_ERR_CAPACITY: return "MOE_ERR_CAPACITY: rows_capacity below T*k + E*(pad-1)";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than moe_workspace_bytes";
    case MOE_ERR_ALIAS: return "MOE_ERR_ALIAS: an output overlaps an input or another output";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: kernel launch failed";
    case MOE_ERR_SCRATCH:
      return "MOE_ERR_SCRATCH: T, E, k need more than the static scratch of "
             "moe_dispatch_noalloc (MOE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown moe_status";
  }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

size_t moe_rows_capacity(int T, int E, int k, int pad) {
  if (check_route_shape(T, E, k, pad) != MOE_OK) return 0;
  return (size_t)T * k + (size_t)E * (pad - 1);
}

size_t moe_workspace_bytes(int T, int E, int k) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK)
    return 0;
  return moe::workspace_bytes(T, E, k);
}

int moe_route(const void* x, int x_dtype, int T, int H, const void* w_gate,
              int E, const float* bias, int k, int pad, int32_t* topk_idx,
              float* topk_w, int32_t* counts, int32_t* offsets,
              float* logits_dbg, void* workspace, size_t workspace_bytes,
              void* stream) {
  int st = check_route_shape(T, E, k, pad);
  if (st != MOE_OK) return st;
  if (H < 8 || H % 8 != 0) return MOE_ERR_SHAPE;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if ((st = check_gate_wide(T, E, x_dtype)) != MOE_OK) return st;
  if (counts == nullptr || offsets == nullptr) return MOE_ERR_NULL;
  if (T > 0 && (x == nullptr || w_gate == nullptr || topk_idx == nullptr ||
                topk_w == nullptr || workspace == nullptr))
    return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(bias, 4) ||
      !aligned(topk_idx, 4) || !aligned(topk_w, 4) || !aligned(counts, 4) ||
      !aligned(offsets, 4) || !aligned(logits_dbg, 4) || !aligned(workspace, 16))
    return MOE_ERR_ALIGN;
  if (workspace_bytes < moe::workspace_bytes(T, E, k)) return MOE_ERR_WORKSPACE;
  const size_t es = dtype_size(x_dtype);
  const Span ins[] = {{x, (size_t)T * H * es}, {w_gate, (size_t)E * H * es},
                      {bias, bias ? (size_t)E * 4 : 0}};
  const Span outs[] = {{topk_idx, (size_t)T * k * 4}, {topk_w, (size_t)T * k * 4},
                       {counts, (size_t)E * 4}, {offsets, (size_t)(E + 1) * 4},
                       {logits_dbg, logits_dbg ? (size_t)T * E * 4 : 0},
                       {workspace, moe::workspace_bytes(T, E, k)}};
  if (any_overlap(outs, 6, ins, 3)) return MOE_ERR_ALIAS;
  if (trace_on())
    std::fprintf(stderr, "moe_route T=%d H=%d E=%d k=%d pad=%d dtype=%d\n", T,
                 H, E, k, pad, x_dtype);
  return hip_status(moe::launch_route(x, w_gate, x_dtype, bias, T, H, E, k,
                                      pad, topk_idx, topk_w, counts, offsets,
                                      logits_dbg, workspace,
                                      (hipStream_t)stream));
}

int moe_plan(const int32_t* topk_idx, int T, int k, int E, int pad,
             int32_t* counts, int32_t* offsets, void* workspace,
             size_t workspace_bytes, void* stream) {
  int st = check_route_shape(T, E, k, pad);
  if (st != MOE_OK) return st;
  if (counts == nullptr || offsets == nullptr) return MOE_ERR_NULL;
  if (T > 0 && (topk_idx == nullptr || workspace == nullptr)) return MOE_ERR_NULL;
  if (!aligned(topk_idx, 4) || !aligned(counts, 4) || !aligned(offsets, 4) ||
      !aligned(workspace, 16))
    return MOE_ERR_ALIGN;
  if (workspace_bytes < moe::workspace_bytes(T, E, k)) return MOE_ERR_WORKSPACE;
  const Span ins[] = {{topk_idx, (size_t)T * k * 4}};
  const Span outs[] = {{counts, (size_t)E * 4}, {offsets, (size_t)(E + 1) * 4},
                       {workspace, moe::workspace_bytes(T, E, k)}};
  if (any_overlap(outs, 3, ins, 1)) return MOE_ERR_ALIAS;
  if (trace_on())
    std::fprintf(stderr, "moe_plan T=%d E=%d k=%d pad=%d\n", T, E, k, pad);
  return hip_status(moe::launch_plan(topk_idx, T, k, E, pad, counts, offsets,
                                     workspace, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Argument checks shared by moe_dispatch (need_ws: a workspace of
// workspace_bytes is one more input) and moe_dispatch_noalloc (none).
int check_dispatch(const void* x, int x_dtype, int T, int H,
                   const int32_t* topk_idx, int k, int E, int pad,
                   const int32_t* counts, const int32_t* offsets,
                   bool need_ws, const void* workspace,
                   size_t workspace_bytes, int payload_dtype, void* rows,
                   size_t rows_capacity, float* row_scales, int32_t* row_src,
                   int32_t* tok_row) {
  int st = check_route_shape(T, E, k, pad);
  if (st != MOE_OK) return st;
  if (H < 8 || H % 8 != 0) return MOE_ERR_SHAPE;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  const bool fp8 = payload_dtype == MOE_FP8_E4M3;
  if (payload_dtype != x_dtype && !fp8) return MOE_ERR_DTYPE;
  if (fp8 && H % 128 != 0) return MOE_ERR_SHAPE;
  if (counts == nullptr || offsets == nullptr || row_src == nullptr)
    return MOE_ERR_NULL;
  if (fp8 != (row_scales != nullptr)) return fp8 ? MOE_ERR_NULL : MOE_ERR_DTYPE;
  if (T > 0 && (x == nullptr || topk_idx == nullptr ||
                (need_ws && workspace == nullptr) || rows == nullptr ||
                tok_row == nullptr))
    return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(rows, 16) || !aligned(topk_idx, 4) ||
      !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(workspace, 16) ||
      !aligned(row_scales, 4) || !aligned(row_src, 4) || !aligned(tok_row, 4))
    return MOE_ERR_ALIGN;
  if (rows_capacity < moe_rows_capacity(T, E, k, pad)) return MOE_ERR_CAPACITY;
  if (rows_capacity > 0x7fffffffULL) return MOE_ERR_SHAPE;
  if (need_ws && workspace_bytes < moe::workspace_bytes(T, E, k))
    return MOE_ERR_WORKSPACE;
  const size_t xs = dtype_size(x_dtype), ps = dtype_size(payload_dtype);
  const Span ins[] = {{x, (size_t)T * H * xs}, {topk_idx, (size_t)T * k * 4},
                      {counts, (size_t)E * 4}, {offsets, (size_t)(E + 1) * 4},
                      {workspace,
                       need_ws ? moe::workspace_bytes(T, E, k) : 0}};
  const Span outs[] = {{rows, rows_capacity * H * ps},
                       {row_scales, fp8 ? rows_capacity * (H / 128) * 4 : 0},
                       {row_src, rows_capacity * 4},
                       {tok_row, (size_t)T * k * 4}};
  if (any_overlap(outs, 4, ins, 5)) return MOE_ERR_ALIAS;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_dispatch(const void* x, int x_dtype, int T, int H,
                 const int32_t* topk_idx, int k, int E, int pad,
                 const int32_t* counts, const int32_t* offsets,
                 const void* workspace, size_t workspace_bytes,
                 int payload_dtype, void* rows, size_t rows_capacity,
                 float* row_scales, int32_t* row_src, int32_t* tok_row,
                 void* stream) {
  const int st = check_dispatch(x, x_dtype, T, H, topk_idx, k, E, pad,
                                counts, offsets, true, workspace,
                                workspace_bytes, payload_dtype, rows,
                                rows_capacity, row_scales, row_src, tok_row);
  if (st != MOE_OK) return st;
  if (trace_on())
    std::fprintf(stderr, "moe_dispatch T=%d H=%d E=%d k=%d payload=%d cap=%zu\n",
                 T, H, E, k, payload_dtype, rows_capacity);
  if (T == 0 && rows_capacity == 0) return MOE_OK;
  return hip_status(moe::launch_dispatch(
      x, x_dtype, T, H, topk_idx, k, E, counts, offsets, workspace,
      payload_dtype, rows, rows_capacity, row_scales, row_src, tok_row,
      (hipStream_t)stream));
}

namespace {
// Arguments of moe_route_dispatch (and of its one-launch form).
int check_route_dispatch(const void* x, int x_dtype, int T, int H,
                         const void* w_gate, int E, const float* bias, int k,
                         int pad, int32_t* topk_idx, float* topk_w,
                         int32_t* counts, int32_t* offsets, float* logits_dbg,
                         void* workspace, size_t workspace_bytes,
                         int payload_dtype, void* rows, size_t rows_capacity,
                         float* row_scales, int32_t* row_src,
                         int32_t* tok_row) {
  int st = check_route_shape(T, E, k, pad);
  if (st != MOE_OK) return st;
  if (H < 8 || H % 8 != 0) return MOE_ERR_SHAPE;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if ((st = check_gate_wide(T, E, x_dtype)) != MOE_OK) return st;
  const bool fp8 = payload_dtype == MOE_FP8_E4M3;
  if (payload_dtype != x_dtype && !fp8) return MOE_ERR_DTYPE;
  if (fp8 && H % 128 != 0) return MOE_ERR_SHAPE;
  if (counts == nullptr || offsets == nullptr || row_src == nullptr)
    return MOE_ERR_NULL;
  if (fp8 != (row_scales != nullptr)) return fp8 ? MOE_ERR_NULL : MOE_ERR_DTYPE;
  if (T > 0 && (x == nullptr || w_gate == nullptr || topk_idx == nullptr ||
                topk_w == nullptr || workspace == nullptr || rows == nullptr ||
                tok_row == nullptr))
    return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(bias, 4) ||
      !aligned(topk_idx, 4) || !aligned(topk_w, 4) || !aligned(counts, 4) ||
      !aligned(offsets, 4) || !aligned(logits_dbg, 4) ||
      !aligned(workspace, 16) || !aligned(rows, 16) ||
      !aligned(row_scales, 4) || !aligned(row_src, 4) || !aligned(tok_row, 4))
    return MOE_ERR_ALIGN;
  if (rows_capacity < moe_rows_capacity(T, E, k, pad)) return MOE_ERR_CAPACITY;
  if (rows_capacity > 0x7fffffffULL) return MOE_ERR_SHAPE;
  if (workspace_bytes < moe::workspace_bytes(T, E, k)) return MOE_ERR_WORKSPACE;
  const size_t es = dtype_size(x_dtype), ps = dtype_size(payload_dtype);
  const Span ins[] = {{x, (size_t)T * H * es}, {w_gate, (size_t)E * H * es},
                      {bias, bias ? (size_t)E * 4 : 0}};
  const Span outs[] = {{topk_idx, (size_t)T * k * 4},
                       {topk_w, (size_t)T * k * 4},
                       {counts, (size_t)E * 4},
                       {offsets, (size_t)(E + 1) * 4},
                       {logits_dbg, logits_dbg ? (size_t)T * E * 4 : 0},
                       {workspace, moe::workspace_bytes(T, E, k)},
                       {rows, rows_capacity * H * ps},
                       {row_scales, fp8 ? rows_capacity * (H / 128) * 4 : 0},
                       {row_src, rows_capacity * 4},
                       {tok_row, (size_t)T * k * 4}};
  if (any_overlap(outs, 10, ins, 3)) return MOE_ERR_ALIAS;
  return MOE_OK;
}
}  // namespace

int moe_route_dispatch(const void* x, int x_dtype, int T, int H,
                       const void* w_gate, int E, const float* bias, int k,
                       int pad, int32_t* topk_idx, float* topk_w,
                       int32_t* counts, int32_t* offsets, float* logits_dbg,
                       void* workspace, size_t workspace_bytes,
                       int payload_dtype, void* rows, size_t rows_capacity,
                       float* row_scales, int32_t* row_src, int32_t* tok_row,
                       void* stream) {
  const int st = check_route_dispatch(
      x, x_dtype, T, H, w_gate, E, bias, k, pad, topk_idx, topk_w, counts,
      offsets, logits_dbg, workspace, workspace_bytes, payload_dtype, rows,
      rows_capacity, row_scales, row_src, tok_row);
  if (st != MOE_OK) return st;
  if (trace_on())
    std::fprintf(stderr,
                 "moe_route_dispatch T=%d H=%d E=%d k=%d pad=%d dtype=%d "
                 "payload=%d cap=%zu\n",
                 T, H, E, k, pad, x_dtype, payload_dtype, rows_capacity);
  return hip_status(moe::launch_route_dispatch(
      x, w_gate, x_dtype, bias, T, H, E, k, pad, topk_idx, topk_w, counts,
      offsets, logits_dbg, workspace, payload_dtype, rows, rows_capacity,
      row_scales, row_src, tok_row, (hipStream_t)stream));
}

int moe_route_dispatch_one_launch(
    const void* x, int x_dtype, int T, int H, const void* w_gate, int E,
    const float* bias, int k, int pad, int32_t* topk_idx, float* topk_w,
    int32_t* counts, int32_t* offsets, float* logits_dbg, void* workspace,
    size_t workspace_bytes, int payload_dtype, void* rows,
    size_t rows_capacity, float* row_scales, int32_t* row_src,
    int32_t* tok_row, void* stream) {
  const int st = check_route_dispatch(
      x, x_dtype, T, H, w_gate, E, bias, k, pad, topk_idx, topk_w, counts,
      offsets, logits_dbg, workspace, workspace_bytes, payload_dtype, rows,
      rows_capacity, row_scales, row_src, tok_row);
  if (st != MOE_OK) return st;
  if (x_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (T > moe::kOneLaunchMaxT || E > moe::kGateWideE) return MOE_ERR_SHAPE;
  if (T == 0)
    return moe_route_dispatch(x, x_dtype, T, H, w_gate, E, bias, k, pad,
                              topk_idx, topk_w, counts, offsets, logits_dbg,
                              workspace, workspace_bytes, payload_dtype, rows,
                              rows_capacity, row_scales, row_src, tok_row,
                              stream);
  if (trace_on())
    std::fprintf(stderr,
                 "moe_route_dispatch_one_launch T=%d H=%d E=%d k=%d pad=%d "
                 "payload=%d cap=%zu\n",
                 T, H, E, k, pad, payload_dtype, rows_capacity);
  return hip_status(moe::launch_route_dispatch_one_launch(
      x, w_gate, bias, T, H, E, k, pad, topk_idx, topk_w, counts, offsets,
      logits_dbg, workspace, payload_dtype, rows, rows_capacity, row_scales,
      row_src, tok_row, (hipStream_t)stream));
}

size_t moe_noalloc_scratch_bytes(int T, int E, int k) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK)
    return 0;
  return moe::noalloc_bytes(T, E, k);
}

int moe_dispatch_noalloc(const void* x, int x_dtype, int T, int H,
                         const int32_t* topk_idx, int k, int E, int pad,
                         const int32_t* counts, const int32_t* offsets,
                         int payload_dtype, void* rows, size_t rows_capacity,
                         float* row_scales, int32_t* row_src,
                         int32_t* tok_row, void* stream) {
  const int st = check_dispatch(x, x_dtype, T, H, topk_idx, k, E, pad,
                                counts, offsets, false, nullptr, 0,
                                payload_dtype, rows, rows_capacity,
                                row_scales, row_src, tok_row);
  if (st != MOE_OK) return st;
  if (moe::noalloc_bytes(T, E, k) > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return MOE_ERR_SCRATCH;
  if (trace_on())
    std::fprintf(stderr,
                 "moe_dispatch_noalloc T=%d H=%d E=%d k=%d payload=%d "
                 "cap=%zu\n",
                 T, H, E, k, payload_dtype, rows_capacity);
  if (T == 0 && rows_capacity == 0) return MOE_OK;
  return hip_status(moe::launch_dispatch_noalloc(
      x, x_dtype, T, H, topk_idx, k, E, pad, counts, offsets, payload_dtype,
      rows, rows_capacity, row_scales, row_src, tok_row, (hipStream_t)stream));
}

int moe_combine_residual(const void* y, int y_dtype, int H, size_t y_rows,
                         const int32_t* tok_row, const float* topk_w, int T,
                         int k, const void* shared, const void* residual_in,
                         void* residual_out, void* residual_no_routed,
                         void* out, int out_dtype, void* stream) {
  if (T < 0 || H < 8 || H % 8 != 0 || k < 1 || k > MOE_MAX_TOPK)
    return MOE_ERR_SHAPE;
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  const bool dual = residual_in != nullptr;
  if (dual) {
    if (residual_out == nullptr) return MOE_ERR_NULL;
    if (out != nullptr) return MOE_ERR_ALIAS;
  } else {
    if (out == nullptr) return MOE_ERR_NULL;
    if (residual_out != nullptr || residual_no_routed != nullptr)
      return MOE_ERR_ALIAS;
    if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  }
  if (T > 0 && (y == nullptr || tok_row == nullptr || topk_w == nullptr))
    return MOE_ERR_NULL;
  if (!aligned(y, 16) || !aligned(shared, 16) || !aligned(residual_in, 16) ||
      !aligned(residual_out, 16) || !aligned(residual_no_routed, 16) ||
      !aligned(out, 16) || !aligned(tok_row, 4) || !aligned(topk_w, 4))
    return MOE_ERR_ALIGN;
  const size_t tb = (size_t)T * H * 2;
  const Span ins[] = {{y, y_rows * H * dtype_size(y_dtype)},
                      {tok_row, (size_t)T * k * 4},
                      {topk_w, (size_t)T * k * 4},
                      {shared, shared ? tb : 0}};
  if (dual) {
    // residual_out may be residual_in itself, but not a partial overlap
    if (residual_out != residual_in &&
        overlap({residual_out, tb}, {residual_in, tb}))
      return MOE_ERR_ALIAS;
    const Span outs[] = {{residual_out, tb}, {residual_no_routed, tb}};
    if (any_overlap(outs, 2, ins, 4)) return MOE_ERR_ALIAS;
    if (overlap({residual_no_routed, tb}, {residual_in, tb})) return MOE_ERR_ALIAS;
  } else {
    const Span outs[] = {{out, (size_t)T * H * dtype_size(out_dtype)}};
    if (any_overlap(outs, 1, ins, 4)) return MOE_ERR_ALIAS;
  }
  if (trace_on())
    std::fprintf(stderr, "moe_combine_residual T=%d H=%d k=%d dual=%d\n", T, H,
                 k, (int)dual);
  if (T == 0) return MOE_OK;
  return hip_status(moe::launch_combine(
      y, y_dtype, H, y_rows, tok_row, topk_w, T, k, shared, residual_in,
      residual_out, residual_no_routed, out, dual ? MOE_BF16 : out_dtype,
      (hipStream_t)stream));
}

int moe_farskip_aux(const void* shared, const void* residual_in,
                    void* residual_no_routed, int T, int H, void* stream) {
  if (T < 0 || H < 8 || H % 8 != 0) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (residual_in == nullptr || residual_no_routed == nullptr)
    return MOE_ERR_NULL;
  if (!aligned(shared, 16) || !aligned(residual_in, 16) ||
      !aligned(residual_no_routed, 16))
    return MOE_ERR_ALIGN;
  const size_t tb = (size_t)T * H * 2;
  const Span ins[] = {{shared, shared ? tb : 0}, {residual_in, tb}};
  const Span outs[] = {{residual_no_routed, tb}};
  if (any_overlap(outs, 1, ins, 2)) return MOE_ERR_ALIAS;
  return hip_status(moe::launch_farskip_aux(shared, residual_in,
                                            residual_no_routed, T, H,
                                            (hipStream_t)stream));
}

int moe_combine_backward(const void* grad_out, const void* y, int y_dtype,
                         int H, size_t y_rows, const int32_t* tok_row,
                         const float* topk_w, int T, int k, void* grad_y,
                         float* grad_w, void* stream) {
  if (T < 0 || H < 8 || H % 8 != 0 || k < 1 || k > MOE_MAX_TOPK)
    return MOE_ERR_SHAPE;
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (grad_out == nullptr || y == nullptr || tok_row == nullptr ||
      topk_w == nullptr || grad_y == nullptr || grad_w == nullptr)
    return MOE_ERR_NULL;
  if (!aligned(grad_out, 16) || !aligned(y, 16) || !aligned(grad_y, 16) ||
      !aligned(tok_row, 4) || !aligned(topk_w, 4) || !aligned(grad_w, 4))
    return MOE_ERR_ALIGN;
  const Span ins[] = {{grad_out, (size_t)T * H * 2},
                      {y, y_rows * H * dtype_size(y_dtype)},
                      {tok_row, (size_t)T * k * 4},
                      {topk_w, (size_t)T * k * 4}};
  const Span outs[] = {{grad_y, y_rows * H * 2}, {grad_w, (size_t)T * k * 4}};
  if (any_overlap(outs, 2, ins, 4)) return MOE_ERR_ALIAS;
  return hip_status(moe::launch_combine_backward(
      grad_out, y, y_dtype, H, y_rows, tok_row, topk_w, T, k, grad_y, grad_w,
      (hipStream_t)stream));
}

int moe_dispatch_backward(const void* grad_rows, int rows_dtype, int H,
                          size_t rows_capacity, const int32_t* tok_row, int T,
                          int k, void* grad_x, int grad_x_dtype,
                          void* stream) {
  if (T < 0 || H < 8 || H % 8 != 0 || k < 1 || k > MOE_MAX_TOPK)
    return MOE_ERR_SHAPE;
  if (rows_dtype != MOE_F32 && rows_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (grad_x_dtype != MOE_F32 && grad_x_dtype != MOE_BF16)
    return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (grad_rows == nullptr || tok_row == nullptr || grad_x == nullptr)
    return MOE_ERR_NULL;
  if (!aligned(grad_rows, 16) || !aligned(grad_x, 16) || !aligned(tok_row, 4))
    return MOE_ERR_ALIGN;
  const Span ins[] = {{grad_rows, rows_capacity * H * dtype_size(rows_dtype)},
                      {tok_row, (size_t)T * k * 4}};
  const Span outs[] = {{grad_x, (size_t)T * H * dtype_size(grad_x_dtype)}};
  if (any_overlap(outs, 1, ins, 2)) return MOE_ERR_ALIAS;
  // an unweighted combine: grad_x[t] = sum_j grad_rows[tok_row[t, j]]
  return hip_status(moe::launch_combine(grad_rows, rows_dtype, H,
                                        rows_capacity, tok_row, nullptr, T, k,
                                        nullptr, nullptr, nullptr, nullptr,
                                        grad_x, grad_x_dtype,
                                        (hipStream_t)stream));
}

size_t moe_expert_gemm_workspace_bytes(size_t rows_capacity, int E) {
  if (E < 1 || E > MOE_MAX_EXPERTS) return 0;
  return moe::gemm_workspace_bytes(rows_capacity, E);
}

int moe_expert_gemm_fp8(const void* rows, const float* row_scales, int K,
                        size_t rows_capacity, const int32_t* row_src,
                        const int32_t* offsets, int E, const void* w,
                        const float* w_scales, int N, void* y, int y_dtype,
                        void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (K < 128 || K % 128 != 0 || K > moe::kGemmMaxK || N < 128 ||
      N % 128 != 0 || E < 1 || E > MOE_MAX_EXPERTS ||
      rows_capacity * (size_t)K > (size_t)0xffffffff ||
      (size_t)N * (size_t)K > (size_t)0xffffffff)
    return MOE_ERR_SHAPE;
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (rows_capacity == 0) return MOE_OK;
  if (rows == nullptr || row_scales == nullptr || offsets == nullptr ||
      w == nullptr || w_scales == nullptr || y == nullptr ||
      workspace == nullptr)
    return MOE_ERR_NULL;
  if (workspace_bytes < moe::gemm_workspace_bytes(rows_capacity, E))
    return MOE_ERR_WORKSPACE;
  if (!aligned(rows, 16) || !aligned(w, 16) || !aligned(y, 16) ||
      !aligned(workspace, 16) || !aligned(row_scales, 4) ||
      !aligned(w_scales, 4) || !aligned(offsets, 4) || !aligned(row_src, 4))
    return MOE_ERR_ALIGN;
  const size_t kb = (size_t)K / 128;
  const Span ins[] = {{rows, rows_capacity * K},
                      {row_scales, rows_capacity * kb * 4},
                      {row_src, row_src ? rows_capacity * 4 : 0},
                      {offsets, (size_t)(E + 1) * 4},
                      {w, (size_t)E * N * K},
                      {w_scales, (size_t)E * (N / 128) * kb * 4}};
  const Span outs[] = {
      {y, rows_capacity * N * dtype_size(y_dtype)},
      {workspace, moe::gemm_workspace_bytes(rows_capacity, E)}};
  if (any_overlap(outs, 2, ins, 6) || overlap(outs[0], outs[1]))
    return MOE_ERR_ALIAS;
  if (trace_on())
    std::fprintf(stderr, "moe_expert_gemm_fp8 cap=%zu K=%d N=%d E=%d\n",
                 rows_capacity, K, N, E);
  return hip_status(moe::launch_expert_gemm(
      rows, row_scales, K, rows_capacity, row_src, offsets, E, w, w_scales, N,
      y, y_dtype, workspace, (hipStream_t)stream));
}

int moe_expert_fixture(const void* rows, int payload_dtype,
                       const float* row_scales, int H, const int32_t* row_src,
                       const int32_t* offsets, int E, const float* sigma,
                       size_t rows_capacity, void* y, int y_dtype,
                       void* stream) {
  if (H < 8 || H % 8 != 0 || E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
  if (payload_dtype < MOE_F32 || payload_dtype > MOE_FP8_E4M3)
    return MOE_ERR_DTYPE;
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  const bool fp8 = payload_dtype == MOE_FP8_E4M3;
  if (fp8 && H % 128 != 0) return MOE_ERR_SHAPE;
  if (rows_capacity == 0) return MOE_OK;
  if (rows == nullptr || row_src == nullptr || offsets == nullptr ||
      sigma == nullptr || y == nullptr || (fp8 && row_scales == nullptr))
    return MOE_ERR_NULL;
  if (!aligned(rows, 16) || !aligned(y, 16)) return MOE_ERR_ALIGN;
  const Span ins[] = {{rows, rows_capacity * H * dtype_size(payload_dtype)}};
  const Span outs[] = {{y, rows_capacity * H * dtype_size(y_dtype)}};
  if (any_overlap(outs, 1, ins, 1)) return MOE_ERR_ALIAS;
  return hip_status(moe::launch_fixture(rows, payload_dtype, row_scales, H,
                                        row_src, offsets, E, sigma,
                                        rows_capacity, y, y_dtype,
                                        (hipStream_t)stream));
}

}  // extern "C"
