// Internal launchers: each enqueues one stage's kernels on `stream`.
// Arguments have been validated by the C-ABI layer (moe_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Histogram tiles of the workspace for T tokens.
inline int num_tiles(int T) { return (T + 63) / 64; }

// Workspace layout (int32 arrays, each 256-byte aligned):
//   tile_base [ntiles, E]  per-tile expert counts, then (after the scan)
//                          the first row of each tile's tokens for expert e
//   slot_rank [T, k]       rank of slot (t, j) among its tile's tokens that
//                          chose the same expert
inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }
inline size_t ws_tile_bytes(int T, int E) {
  return align256(size_t(num_tiles(T)) * size_t(E) * 4);
}
inline size_t ws_rank_bytes(int T, int k) {
  return align256(size_t(T) * size_t(k) * 4);
}
inline size_t workspace_bytes(int T, int E, int k) {
  return T == 0 ? 0 : ws_tile_bytes(T, E) + ws_rank_bytes(T, k);
}

// dtype codes of moe.h
enum { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

// gate + top-k + tile histogram + scan (the whole of moe_route)
hipError_t launch_route(const void* x, const void* w, int xdt,
                        const float* bias, int T, int H, int E, int k,
                        int pad, int32_t* topk_idx, float* topk_w,
                        int32_t* counts, int32_t* offsets, float* logits_dbg,
                        void* workspace, hipStream_t s);

hipError_t launch_plan(const int32_t* topk_idx, int T, int k, int E, int pad,
                       int32_t* counts, int32_t* offsets, void* workspace,
                       hipStream_t s);

hipError_t launch_dispatch(const void* x, int xdt, int T, int H,
                           const int32_t* topk_idx, int k, int E,
                           const int32_t* counts, const int32_t* offsets,
                           const void* workspace, int pdt, void* rows,
                           size_t capacity, float* row_scales,
                           int32_t* row_src, int32_t* tok_row, hipStream_t s);

hipError_t launch_combine(const void* y, int ydt, int H, size_t y_rows,
                          const int32_t* tok_row, const float* topk_w, int T,
                          int k, const void* shared, const void* res_in,
                          void* res_out, void* rnr, void* out, int odt,
                          hipStream_t s);

hipError_t launch_fixture(const void* rows, int pdt, const float* row_scales,
                          int H, const int32_t* row_src,
                          const int32_t* offsets, int E, const float* sigma,
                          size_t capacity, void* y, int ydt, hipStream_t s);

}  // namespace moe
