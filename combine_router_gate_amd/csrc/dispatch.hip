// Stable scatter of token rows into the expert-major buffer padded per
// expert, optionally quantised to OCP fp8 E4M3 with one fp32 scale per
// 1x128 block, for gfx950.
//
// Tokens are copied into contiguous per-expert buffers that feed the
// experts, and the row every (token, slot) copy went to is recorded for the
// combine ("Efficient and Portable Mixture-of-Experts Communication",
// sections Dispatch and Combine); fp8 tokens travel with their block scaling
// factors (same page, Dispatch).  That design hands out receive rows with an
// atomically incremented counter, so its order varies run to run; here the
// row of slot (t, j) is fixed by the scan: row = first row of (tile(t), e)
// + rank of t among the tile's tokens that chose e, i.e. ascending token
// order inside every expert segment.
//
// Design for CDNA4: a token's row is split into groups of 64-lane chunks
// (two chunks per lane, or one with few tokens), one wavefront each, so the
// waves of a token run side by side.  Lanes 0..k-1 resolve the k
// destination rows, which are then broadcast to scalar registers; the token
// row is read from HBM once in 16-byte vectors (coalesced across the wave)
// and written k times with streaming (non-temporal) stores, which measured
// ~20% faster than cached stores for this write-dominated scatter.  The fp8
// path gives each 128-element block to an aligned group of 8 lanes (16
// elements per lane): the block's absolute max is an 8-lane reduction, the
// scale and quotients are IEEE fp32 divisions, the codes come from the
// hardware E4M3 converter, and each lane writes 16 code bytes per
// destination.  Extra workgroups mark padding rows (row_src = -1) in the
// same launch.
#include "scatter_device.h"

namespace moe {

template <int KMAX, int MODE, int U>
__global__ __launch_bounds__(256) void dispatch_kernel(
    const unsigned char* __restrict__ x, int esize, int T, int H,
    const int32_t* __restrict__ topk_idx, int k, int E,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_base,
    const int32_t* __restrict__ slot_rank, unsigned char* __restrict__ rows,
    long long capacity, float* __restrict__ row_scales,
    int32_t* __restrict__ row_src, int32_t* __restrict__ tok_row,
    int tok_blocks, int hsplit) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if ((int)blockIdx.x >= tok_blocks) {
    fill_padding_rows(blockIdx.x - tok_blocks, kDispatchFillBlocks, E, counts,
                      offsets, capacity, row_src);
    return;
  }
  // wave -> (token, part): hsplit waves share one token's row (interleaved
  // groups of 64-lane chunks); part 0 writes the metadata
  const int gw = blockIdx.x * 4 + wv;
  const int t = gw / hsplit, part = gw - t * hsplit;
  if (t >= T) return;
  const int r =
      token_row(t, lane, k, E, capacity, topk_idx, tile_base, slot_rank);
  int rj[KMAX];
  publish_rows<KMAX>(r, t, part, lane, k, row_src, tok_row, rj);
  scatter_token_part<KMAX, MODE, U>(x, esize, H, t, part, hsplit, lane, rj,
                                    rows, row_scales);
}

// ------------------------------------------------------------------ small batches

// Plan and scatter of few tokens in one launch (the launch after the top-k):
// every workgroup rebuilds the plan in LDS from topk_idx -- no plan kernel
// between top-k and scatter -- then runs its share of the scatter waves or
// of the padding fill; workgroup 0 also stores counts and offsets.
template <int KMAX, int MODE, int U>
__global__ __launch_bounds__(256) void plan_dispatch_small_kernel(
    const unsigned char* __restrict__ x, int esize, int T, int H,
    const int32_t* __restrict__ topk_idx, int k, int E, int pad,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    unsigned char* __restrict__ rows, long long capacity,
    float* __restrict__ row_scales, int32_t* __restrict__ row_src,
    int32_t* __restrict__ tok_row, int tok_blocks, int hsplit) {
  extern __shared__ unsigned long long plan_lds[];
  LocalPlan p = local_plan_arrays(plan_lds, T, E);
  local_plan(topk_idx, T, k, E, pad, p.bits, p.base, p.cnt, p.off);
  plan_dispatch_block<KMAX, MODE, U>(blockIdx.x, x, esize, T, H, topk_idx, k,
                                     E, counts, offsets, rows, capacity,
                                     row_scales, row_src, tok_row, tok_blocks,
                                     hsplit, p);
}

// ------------------------------------------------------------------ fixture

// Stand-in expert for tests and benchmarks: y[r] = sigma[e] * deq(rows[r]).
// PT: payload 0 f32, 1 bf16, 2 fp8.  YT: output 0 f32, 1 bf16.
template <int PT, int YT>
__global__ __launch_bounds__(256) void fixture_kernel(
    const unsigned char* __restrict__ rows, const float* __restrict__ scales,
    int H, const int32_t* __restrict__ row_src,
    const int32_t* __restrict__ offsets, int E,
    const float* __restrict__ sigma, long long capacity,
    unsigned char* __restrict__ y) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long long r = (long long)blockIdx.x * 4 + wv;
  if (r >= capacity) return;
  const int src = row_src[r];
  const int nc8 = H / 8;
  const size_t ybytes = YT == 0 ? 4 : 2;
  unsigned char* yrow = y + (size_t)r * H * ybytes;
  if (src < 0) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int c = lane; c < nc8; c += 64) {
      st16(yrow + (size_t)c * 8 * ybytes, z);
      if (YT == 0) st16(yrow + (size_t)c * 32 + 16, z);
    }
    return;
  }
  // expert whose segment holds r: the last e with offsets[e] <= r
  int lo = 0, hi = E;                       // invariant offsets[lo] <= r
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  const float sg = sigma[lo];
  for (int c = lane; c < nc8; c += 64) {
    float f[8];
    if constexpr (PT == 0) {
      const unsigned char* p = rows + (size_t)r * H * 4 + (size_t)c * 32;
      const u32x4 v0 = ld16(p), v1 = ld16(p + 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = __uint_as_float(v0[i]);
        f[4 + i] = __uint_as_float(v1[i]);
      }
    } else if constexpr (PT == 1) {
      unpack8_bf16(ld16(rows + (size_t)r * H * 2 + (size_t)c * 16), f);
    } else {
      const u32x2 q =
          *reinterpret_cast<const u32x2*>(rows + (size_t)r * H + (size_t)c * 8);
      const float s = scales[(size_t)r * (H / kFp8Block) + c / 16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = e4m3_decode((q.x >> (8 * i)) & 0xffu) * s;
        f[4 + i] = e4m3_decode((q.y >> (8 * i)) & 0xffu) * s;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = sg * f[i];
    if constexpr (YT == 0) {
      u32x4 v0, v1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v0[i] = __float_as_uint(f[i]);
        v1[i] = __float_as_uint(f[4 + i]);
      }
      st16(yrow + (size_t)c * 32, v0);
      st16(yrow + (size_t)c * 32 + 16, v1);
    } else {
      st16(yrow + (size_t)c * 16, pack8_bf16(f));
    }
  }
}

// ------------------------------------------------------------------ launchers

template <int KMAX, int U>
static void launch_dispatch_k(int mode, dim3 grid, hipStream_t s,
                              const unsigned char* x, int esize, int T, int H,
                              const int32_t* idx, int k, int E,
                              const int32_t* counts, const int32_t* offsets,
                              const int32_t* tb, const int32_t* sr,
                              unsigned char* rows, long long cap, float* sc,
                              int32_t* row_src, int32_t* tok_row, int tblocks,
                              int hs) {
  if (mode == 0)
    hipLaunchKernelGGL((dispatch_kernel<KMAX, 0, U>), grid, dim3(256), 0, s, x,
                       esize, T, H, idx, k, E, counts, offsets, tb, sr, rows,
                       cap, sc, row_src, tok_row, tblocks, hs);
  else if (mode == 1)
    hipLaunchKernelGGL((dispatch_kernel<KMAX, 1, U>), grid, dim3(256), 0, s, x,
                       esize, T, H, idx, k, E, counts, offsets, tb, sr, rows,
                       cap, sc, row_src, tok_row, tblocks, hs);
  else
    hipLaunchKernelGGL((dispatch_kernel<KMAX, 2, U>), grid, dim3(256), 0, s, x,
                       esize, T, H, idx, k, E, counts, offsets, tb, sr, rows,
                       cap, sc, row_src, tok_row, tblocks, hs);
}

hipError_t launch_dispatch(const void* x, int xdt, int T, int H,
                           const int32_t* topk_idx, int k, int E,
                           const int32_t* counts, const int32_t* offsets,
                           const void* workspace, int pdt, void* rows,
                           size_t capacity, float* row_scales,
                           int32_t* row_src, int32_t* tok_row, hipStream_t s) {
  const int32_t* tb = (const int32_t*)workspace;
  const int32_t* sr =
      (const int32_t*)((const unsigned char*)workspace + ws_tile_bytes(T, E));
  const ScatterShape g = scatter_shape(xdt, pdt, T, H);
  const dim3 grid(g.tblocks + kDispatchFillBlocks);
  const unsigned char* xb = (const unsigned char*)x;
  unsigned char* rb = (unsigned char*)rows;
  const long long cap = (long long)capacity;
#define MOE_DISPATCH_K(KV)                                                   \
  do {                                                                       \
    if (g.u == 2)                                                            \
      launch_dispatch_k<KV, 2>(g.mode, grid, s, xb, g.esize, T, H, topk_idx, \
                               k, E, counts, offsets, tb, sr, rb, cap,       \
                               row_scales, row_src, tok_row, g.tblocks,      \
                               g.hs);                                        \
    else                                                                     \
      launch_dispatch_k<KV, 1>(g.mode, grid, s, xb, g.esize, T, H, topk_idx, \
                               k, E, counts, offsets, tb, sr, rb, cap,       \
                               row_scales, row_src, tok_row, g.tblocks,      \
                               g.hs);                                        \
  } while (0)
  if (k <= 1) MOE_DISPATCH_K(1);
  else if (k <= 2) MOE_DISPATCH_K(2);
  else if (k <= 4) MOE_DISPATCH_K(4);
  else if (k <= 8) MOE_DISPATCH_K(8);
  else MOE_DISPATCH_K(16);
#undef MOE_DISPATCH_K
  return hipGetLastError();
}

hipError_t launch_plan_dispatch_small(const void* x, int xdt, int T, int H,
                                      const int32_t* topk_idx, int k, int E,
                                      int pad, int32_t* counts,
                                      int32_t* offsets, int pdt, void* rows,
                                      size_t capacity, float* row_scales,
                                      int32_t* row_src, int32_t* tok_row,
                                      hipStream_t s) {
  // one 64-lane chunk per lane step: few tokens spread over more waves
  const ScatterShape g = scatter_shape(xdt, pdt, T, H, false);
  const dim3 grid(g.tblocks + kDispatchFillBlocks);
  const size_t lds = local_plan_lds_bytes(T, E);
  const unsigned char* xb = (const unsigned char*)x;
  unsigned char* rb = (unsigned char*)rows;
  const long long cap = (long long)capacity;
#define MOE_PDS(KV, MV, UV)                                                   \
  hipLaunchKernelGGL((plan_dispatch_small_kernel<KV, MV, UV>), grid,          \
                     dim3(256), lds, s, xb, g.esize, T, H, topk_idx, k, E,    \
                     pad, counts, offsets, rb, cap, row_scales, row_src,      \
                     tok_row, g.tblocks, g.hs)
#define MOE_PDS_M(KV)                                                         \
  do {                                                                        \
    if (g.mode == 0) MOE_PDS(KV, 0, 1);                                       \
    else if (g.mode == 1) MOE_PDS(KV, 1, 1);                                  \
    else MOE_PDS(KV, 2, 1);                                                   \
  } while (0)
  if (k <= 1) MOE_PDS_M(1);
  else if (k <= 2) MOE_PDS_M(2);
  else if (k <= 4) MOE_PDS_M(4);
  else if (k <= 8) MOE_PDS_M(8);
  else MOE_PDS_M(16);
#undef MOE_PDS_M
#undef MOE_PDS
  return hipGetLastError();
}

hipError_t launch_fixture(const void* rows, int pdt, const float* row_scales,
                          int H, const int32_t* row_src,
                          const int32_t* offsets, int E, const float* sigma,
                          size_t capacity, void* y, int ydt, hipStream_t s) {
  const dim3 grid((unsigned)((capacity + 3) / 4));
  const unsigned char* rb = (const unsigned char*)rows;
  unsigned char* yb = (unsigned char*)y;
  const long long cap = (long long)capacity;
#define MOE_FIX(PV, YV)                                                       \
  hipLaunchKernelGGL((fixture_kernel<PV, YV>), grid, dim3(256), 0, s, rb,     \
                     row_scales, H, row_src, offsets, E, sigma, cap, yb)
  const int pt = pdt == DT_F32 ? 0 : (pdt == DT_BF16 ? 1 : 2);
  const int yt = ydt == DT_F32 ? 0 : 1;
  if (pt == 0 && yt == 0) MOE_FIX(0, 0);
  else if (pt == 0) MOE_FIX(0, 1);
  else if (pt == 1 && yt == 0) MOE_FIX(1, 0);
  else if (pt == 1) MOE_FIX(1, 1);
  else if (yt == 0) MOE_FIX(2, 0);
  else MOE_FIX(2, 1);
#undef MOE_FIX
  return hipGetLastError();
}

}  // namespace moe
