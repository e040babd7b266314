// Wave-level scan shared by the plan kernels (route, dispatch, expert GEMM
// tile map).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe.h"

namespace moe {

// Exclusive scan over vals[0 .. n-1] (LDS, n <= 64 * MAXPER) by one wave,
// in place: lane l owns the contiguous run [l * per, l * per + per) with
// per = ceil(n / 64), so all 64 lanes take part, every load is issued before
// the one shuffle scan of the lane sums, and the latency is that of one LDS
// round trip and one scan whatever n is.  dst, if not NULL, receives the
// same prefixes.  Returns the total (in every lane).
template <int MAXPER>
__device__ __forceinline__ int wave_exclusive_scan(int* vals, int n,
                                                   int32_t* dst) {
  const int lane = threadIdx.x & 63;
  const int per = (n + 63) / 64;
  int loc[MAXPER];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < MAXPER; ++i) {
    const int e = lane * per + i;
    loc[i] = i < per && e < n ? vals[e] : 0;
    sum += loc[i];
  }
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  int run = incl - sum;
#pragma unroll
  for (int i = 0; i < MAXPER; ++i) {
    const int e = lane * per + i;
    if (i < per && e < n) {
      vals[e] = run;
      if (dst != nullptr) dst[e] = run;
    }
    run += loc[i];
  }
  return __shfl(incl, 63, 64);
}

}  // namespace moe
