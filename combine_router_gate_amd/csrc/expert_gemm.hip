// fp8 grouped GEMM over the expert-major buffer (gfx950).
//
// Between dispatch and combine each expert runs its grouped GEMM over its
// contiguous segment of received tokens ("Efficient and Portable
// Mixture-of-Experts Communication", Dispatch: tokens are packed per expert
// for the grouped GEMM; Combine reads its 16-bit outputs).  DeepEP sends
// those tokens as FP8 with block scaling factors (DeepEP news, technical
// overview).  This kernel consumes that layout directly:
//
//   y[r, n] = sum_b sa[r, b] * sw[e, n/128, b] * sum_{h in block b}
//             E4M3(rows[r, h]) * E4M3(w[e, n, h])
//
// for every row r of expert e's segment [offsets[e], offsets[e+1]), with the
// 1x128 activation scales written by dispatch and 128x128 weight blocks.
//
// Design for CDNA4:
//  * v_mfma_scale_f32_16x16x128_f8f6f4 with unit (E8M0 = 1) scales: one
//    instruction is exactly one 128-wide scale block of one 16x16 tile, so
//    its fp32 result is scaled once (row scale x weight scale) and added to
//    the accumulator, the per-block promotion fp8 block scaling needs.
//  * The weight tile is the instruction's first operand, so each lane ends
//    up with 4 consecutive output columns of one row: one row scale per
//    lane and block, 8-byte bf16 stores.
//  * A workgroup computes a 128x128 tile (4 waves of 64x64, 16 MFMAs per
//    block), operands loaded straight into registers one block ahead.
//  * Work order is XCD-aware: consecutive tiles (8 column tiles of one row
//    tile, then the next row tile) are given to workgroups of the same XCD,
//    which then share operands in that XCD's L2.
//  * Row tiles come from a tile map built on the device from offsets, so no
//    count ever returns to the host.

#include "expert_gemm.h"
#include "moe_device.h"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// tiles[mt] = (expert, first row) for every 128-row tile of the padded
// expert segments, (-1, 0) for the unused entries up to mt_ub.  Offsets are
// clamped to the buffer so a corrupt plan cannot address past it.
__global__ __launch_bounds__(512) void gemm_tile_map_kernel(
    const int32_t* __restrict__ offsets, int E, int cap, int mt_ub,
    int2* __restrict__ tiles) {
  __shared__ int off[MOE_MAX_EXPERTS + 1];
  __shared__ int start[MOE_MAX_EXPERTS + 1];
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += 512) {
    const int o = offsets[e];
    off[e] = o < 0 ? 0 : o > cap ? cap : o;
  }
  __syncthreads();
  if (tid < 64) {
    constexpr int PER = MOE_MAX_EXPERTS / 64;
    int loc[PER];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid * PER + i;
      const int seg = e < E ? off[e + 1] - off[e] : 0;
      loc[i] = seg > 0 ? (seg + kGemmTile - 1) / kGemmTile : 0;
      sum += loc[i];
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (tid >= d) incl += o;
    }
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid * PER + i;
      if (e < E) start[e] = run;
      run += loc[i];
    }
    if (tid == 63) start[E] = incl;
  }
  __syncthreads();
  const int total = start[E];
  for (int mt = tid; mt < mt_ub; mt += 512)
    if (mt >= total) tiles[mt] = make_int2(-1, 0);
  for (int e = tid; e < E; e += 512)
    for (int j = 0; start[e] + j < start[e + 1]; ++j)
      if (start[e] + j < mt_ub)
        tiles[start[e] + j] = make_int2(e, off[e] + j * kGemmTile);
}

// Operand fragment of 16 rows x 128 bytes: lane l holds bytes
// [32 * (l / 16), +32) of row l % 16.  Both operands use the same byte
// assignment, so the instruction's sum covers the block's 128 products.
__device__ __forceinline__ i32x8 frag_ld(const unsigned char* p) {
  const u32x4 a = ld16(p), b = ld16(p + 16);
  return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w,
               (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

template <int YT>
__global__ __launch_bounds__(256, 2) void expert_gemm_fp8_kernel(
    const unsigned char* __restrict__ rows, const float* __restrict__ rscale,
    int K, int cap, const int32_t* __restrict__ row_src,
    const int32_t* __restrict__ offsets, const unsigned char* __restrict__ w,
    const float* __restrict__ wscale, int N, unsigned char* __restrict__ y,
    const int2* __restrict__ tiles, int mt_ub, int ntn, int gn,
    int per_xcd) {
  __shared__ float sa[kGemmMaxK];          // [block][row of the tile]
  __shared__ float sw[kGemmMaxK / 128];    // [block]
  const int bid = blockIdx.x;
  const int wi = (bid & 7) * per_xcd + (bid >> 3);
  const int ng = wi / (mt_ub * gn);
  const int rem = wi - ng * mt_ub * gn;
  const int mt = rem / gn;
  const int nt = ng * gn + (rem - mt * gn);
  if (mt >= mt_ub || nt >= ntn) return;
  const int2 tile = tiles[mt];
  const int e = tile.x;
  if (e < 0) return;
  const int r0 = tile.y;
  int r_end = offsets[e + 1];
  r_end = r_end > cap ? cap : r_end;
  r_end = r_end < r0 + kGemmTile ? r_end : r0 + kGemmTile;
  if (r_end <= r0) return;
  const int KB = K / 128;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int m0 = 64 * (wv & 1), n0 = 64 * (wv >> 1);

  for (int i = tid; i < kGemmTile * KB; i += 256) {
    const int row = i / KB, b = i - row * KB;
    const int r = r0 + row < r_end ? r0 + row : r_end - 1;
    sa[b * kGemmTile + row] = rscale[(size_t)r * KB + b];
  }
  const float* swp = wscale + ((size_t)e * (N / 128) + nt) * KB;
  for (int b = tid; b < KB; b += 256) sw[b] = swp[b];
  __syncthreads();

  const unsigned char* ap[4];
  const unsigned char* bp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int r = r0 + m0 + 16 * i + c16;
    r = r < r_end ? r : r_end - 1;
    ap[i] = rows + (size_t)r * K + 32 * g;
    const int n = nt * kGemmTile + n0 + 16 * i + c16;
    bp[i] = w + ((size_t)e * N + n) * K + 32 * g;
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  i32x8 fa0[4], fb0[4], fa1[4], fb1[4];
  auto load = [&](i32x8 (&fa)[4], i32x8 (&fb)[4], int b) {
    const size_t o = (size_t)b * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[i] = frag_ld(ap[i] + o);
      fb[i] = frag_ld(bp[i] + o);
    }
  };
  auto step = [&](const i32x8 (&fa)[4], const i32x8 (&fb)[4], int b) {
    const float swb = sw[b];
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = sa[b * kGemmTile + m0 + 16 * i + c16] * swb;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            fb[j], fa[i], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(p[q], s[i], acc[i][j][q]);
      }
  };
  load(fa0, fb0, 0);
  for (int b = 0; b < KB; b += 2) {
    // blocks b (buffer 0) and b + 1 (buffer 1); loads stay one block ahead
    // and are clamped to the last block so they are never conditional
    load(fa1, fb1, b + 1 < KB ? b + 1 : KB - 1);
    step(fa0, fb0, b);
    load(fa0, fb0, b + 2 < KB ? b + 2 : KB - 1);
    if (b + 1 < KB) step(fa1, fb1, b + 1);
  }

  // lane: row m0 + 16 i + c16, columns n0 + 16 j + 4 g .. + 3
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + m0 + 16 * i + c16;
    if (r >= r_end) continue;
    const bool live = row_src == nullptr || row_src[r] >= 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t n = (size_t)nt * kGemmTile + n0 + 16 * j + 4 * g;
      f32x4 v = acc[i][j];
      if (!live) v = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (YT == 1) {
        const u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2*>(y + ((size_t)r * N + n) * 2) = pk;
      } else {
        *reinterpret_cast<f32x4*>(y + ((size_t)r * N + n) * 4) = v;
      }
    }
  }
}

hipError_t launch_expert_gemm(const void* rows, const float* row_scales,
                              int K, size_t rows_capacity,
                              const int32_t* row_src, const int32_t* offsets,
                              int E, const void* w, const float* w_scales,
                              int N, void* y, int y_dtype, void* workspace,
                              hipStream_t s) {
  const long long mt_ub = gemm_row_tiles(rows_capacity, E);
  int2* tiles = (int2*)workspace;
  const int cap = (int)rows_capacity;
  hipLaunchKernelGGL(gemm_tile_map_kernel, dim3(1), dim3(512), 0, s, offsets,
                     E, cap, (int)mt_ub, tiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int ntn = N / kGemmTile;
  const int gn = ntn < 8 ? ntn : 8;
  const long long total = (long long)((ntn + gn - 1) / gn) * mt_ub * gn;
  const long long grid = (total + 7) / 8 * 8;
  const int per_xcd = (int)(grid / 8);
  const unsigned char* rb = (const unsigned char*)rows;
  const unsigned char* wb = (const unsigned char*)w;
  unsigned char* yb = (unsigned char*)y;
  if (y_dtype == MOE_BF16)
    hipLaunchKernelGGL((expert_gemm_fp8_kernel<1>), dim3((unsigned)grid),
                       dim3(256), 0, s, rb, row_scales, K, cap, row_src,
                       offsets, wb, w_scales, N, yb, tiles, (int)mt_ub, ntn,
                       gn, per_xcd);
  else
    hipLaunchKernelGGL((expert_gemm_fp8_kernel<0>), dim3((unsigned)grid),
                       dim3(256), 0, s, rb, row_scales, K, cap, row_src,
                       offsets, wb, w_scales, N, yb, tiles, (int)mt_ub, ntn,
                       gn, per_xcd);
  return hipGetLastError();
}

}  // namespace moe
