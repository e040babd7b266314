// Internal launchers: each enqueues one stage's kernels on `stream`.
// Arguments have been validated by the C-ABI layer (moe_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Histogram tiles of the workspace for T tokens.
inline int num_tiles(int T) { return (int)(((long long)T + 63) / 64); }

// Workspace layout (each array 256-byte aligned):
//   tile_base [ntiles, E] int32  per-tile expert counts, then (after the
//                                scan) the first row of each tile's tokens
//                                for expert e
//   slot_rank [T, k] int32       rank of slot (t, j) among its tile's tokens
//                                that chose the same expert
//   partial   [S, T, EP] fp32    partial gate logits when the hidden
//                                dimension is split S ways (up to
//                                kSplitMaxT tokens); S <= split_max(T), EP =
//                                experts padded to the gate's 64 * EPW
//   group     [G, E] int32       per-group expert totals of the parallel
//                                scan (G = ceil(tiles / 16), up to
//                                kSplitMaxT tokens)
inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }
constexpr int kSplitRows = 16384;
constexpr int kSplitMax = 64;
constexpr int kSplitMaxT = 65536;      // more tokens: the one-pass gate
inline int gate_epw(int E) {           // expert tiles per wave of the gate
  const int et = (E + 15) / 16;
  return et <= 4 ? 1 : et <= 8 ? 2 : et <= 16 ? 4 : et <= 24 ? 6
       : et <= 32 ? 8 : et <= 48 ? 12 : 16;
}
// Above this many experts the gate runs only the split bf16 path (partial
// logits in expert groups, a 64-lane top-k per token), so x must be bf16
// and T at most kSplitMaxT (where the workspace holds partial logits).
constexpr int kGateWideE = 512;
// Largest split of H for T tokens: 2 * kSplitRows partial rows, at least 4
// ranges up to kSplitMaxT tokens.
inline int split_max(int T) {
  if (T <= 0 || T > kSplitMaxT) return 1;
  const int s = 2 * kSplitRows / T;
  return s < 4 ? 4 : s < kSplitMax ? s : kSplitMax;
}
inline size_t ws_tile_bytes(int T, int E) {
  return align256(size_t(num_tiles(T)) * size_t(E) * 4);
}
inline size_t ws_rank_bytes(int T, int k) {
  return align256(size_t(T) * size_t(k) * 4);
}
// fp32 partial gate logits of up to split_max(T) hidden ranges
inline size_t ws_partial_bytes(int T, int E) {
  const int s = split_max(T);
  return s > 1 ? align256(size_t(s) * T * 64 * gate_epw(E) * 4) : 0;
}
// Up to this many tokens, histogram, scan and ranks run in one workgroup.
constexpr int kSmallPlanT = 512;
// Tiles per group of the parallel scan: the histogram producers of a split
// gate add each tile's expert counts into its group's totals
// [ceil(tiles / kScanGroup), E] int32 (zeroed by the gate kernel of the
// same call), so one scan workgroup per group needs no other group's tiles.
constexpr int kScanGroup = 16;
inline int num_groups(int T) {
  return (num_tiles(T) + kScanGroup - 1) / kScanGroup;
}
inline size_t ws_group_bytes(int T, int E) {
  return T > 0 && T <= kSplitMaxT
             ? align256(size_t(num_groups(T)) * size_t(E) * 4)
             : 0;
}
inline size_t workspace_bytes(int T, int E, int k) {
  return T == 0 ? 0
                : ws_tile_bytes(T, E) + ws_rank_bytes(T, k) +
                      ws_partial_bytes(T, E) + ws_group_bytes(T, E);
}

// Bytes of the static scratch moe_dispatch_noalloc uses: the workspace's
// tile bases and ranks, then a plan's own counts and offsets.
inline size_t noalloc_bytes(int T, int E, int k) {
  return ws_tile_bytes(T, E) + ws_rank_bytes(T, k) + align256(size_t(E) * 4) +
         align256(size_t(E + 1) * 4);
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

// Plan and scatter of T <= kSmallPlanT tokens in one launch (each workgroup
// rebuilds the plan in LDS from topk_idx; counts and offsets are written)
hipError_t launch_plan_dispatch_small(const void* x, int xdt, int T, int H,
                                      const int32_t* topk_idx, int k, int E,
                                      int pad, int32_t* counts,
                                      int32_t* offsets, int pdt, void* rows,
                                      size_t capacity, float* row_scales,
                                      int32_t* row_src, int32_t* tok_row,
                                      hipStream_t s);

// moe_route followed by moe_dispatch; few tokens without a plan kernel
hipError_t launch_route_dispatch(const void* x, const void* w, int xdt,
                                 const float* bias, int T, int H, int E,
                                 int k, int pad, int32_t* topk_idx,
                                 float* topk_w, int32_t* counts,
                                 int32_t* offsets, float* logits_dbg,
                                 void* workspace, int pdt, void* rows,
                                 size_t capacity, float* row_scales,
                                 int32_t* row_src, int32_t* tok_row,
                                 hipStream_t s);

// moe_route_dispatch in one launch for T <= kOneLaunchMaxT bf16 tokens and
// E <= kGateWideE (grid-wide waits between gate, top-k and scatter)
constexpr int kOneLaunchMaxT = 256;
hipError_t launch_route_dispatch_one_launch(
    const void* x, const void* w, const float* bias, int T, int H, int E,
    int k, int pad, int32_t* topk_idx, float* topk_w, int32_t* counts,
    int32_t* offsets, float* logits_dbg, void* workspace, int pdt, void* rows,
    size_t capacity, float* row_scales, int32_t* row_src, int32_t* tok_row,
    hipStream_t s);

// moe_dispatch with its tile plan rebuilt in the library's static scratch
hipError_t launch_dispatch_noalloc(const void* x, int xdt, int T, int H,
                                   const int32_t* topk_idx, int k, int E,
                                   int pad, const int32_t* counts,
                                   const int32_t* offsets, int pdt, void* rows,
                                   size_t capacity, float* row_scales,
                                   int32_t* row_src, int32_t* tok_row,
                                   hipStream_t s);

hipError_t launch_combine(const void* y, int ydt, int H, size_t y_rows,
                          const int32_t* tok_row, const float* topk_w, int T,
                          int k, const void* shared, const void* res_in,
                          void* res_out, void* rnr, void* out, int odt,
                          hipStream_t s);

hipError_t launch_farskip_aux(const void* shared, const void* residual,
                              void* rnr, int T, int H, hipStream_t s);

hipError_t launch_combine_backward(const void* g, const void* y, int ydt,
                                   int H, size_t y_rows,
                                   const int32_t* tok_row,
                                   const float* topk_w, int T, int k,
                                   void* grad_y, float* grad_w,
                                   hipStream_t s);

hipError_t launch_fixture(const void* rows, int pdt, const float* row_scales,
                          int H, const int32_t* row_src,
                          const int32_t* offsets, int E, const float* sigma,
                          size_t capacity, void* y, int ydt, hipStream_t s);

}  // namespace moe
