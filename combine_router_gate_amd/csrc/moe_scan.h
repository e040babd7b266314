// Wave-level scan shared by the plan kernels (route, dispatch, expert GEMM
// tile map).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

// Exclusive scan over vals[0 .. n-1] (LDS) by one wave, in place: chunks of
// 64 values, one per lane, an inclusive wave scan per chunk plus the running
// carry, so the work follows n and every store is coalesced.  dst, if not
// NULL, receives the same prefixes.  Returns the total (in every lane).
__device__ __forceinline__ int wave_exclusive_scan(int* vals, int n,
                                                   int32_t* dst) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int i = c0 + lane;
    const int v = i < n ? vals[i] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (i < n) {
      vals[i] = carry + incl - v;
      if (dst != nullptr) dst[i] = carry + incl - v;
    }
    carry += __shfl(incl, 63, 64);
  }
  return carry;
}

}  // namespace moe
