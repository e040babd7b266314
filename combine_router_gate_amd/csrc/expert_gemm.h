// Launcher of the fp8 grouped GEMM that stands in for the experts between
// dispatch and combine.  Arguments have been validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kGemmRowsPerTile = 256;   // output rows per workgroup tile
constexpr int kGemmMaxK = 8192;

// Upper bound on the row tiles of all expert segments: each segment has at
// most one partial tile.
inline long long gemm_row_tiles(size_t rows_capacity, int E) {
  return (long long)((rows_capacity + kGemmRowsPerTile - 1) / kGemmRowsPerTile) + E;
}
inline size_t gemm_workspace_bytes(size_t rows_capacity, int E) {
  return ((size_t)gemm_row_tiles(rows_capacity, E) * 8 + 255) & ~size_t(255);
}

hipError_t launch_expert_gemm(const void* rows, const float* row_scales,
                              int K, size_t rows_capacity,
                              const int32_t* row_src, const int32_t* offsets,
                              int E, const void* w, const float* w_scales,
                              int N, void* y, int y_dtype, void* workspace,
                              hipStream_t s);

}  // namespace moe
