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
//  * A workgroup computes a 128x256 tile with 8 waves (two per SIMD, 64x64
//    each; 256-row tiles need more registers than a wave has and spill);
//    operands are staged through two LDS stages, loaded through registers
//    (direct global->LDS copies measured slower on this part).  Global
//    loads are coalesced (8 lanes per 128-byte row segment; with one row
//    per lane the address unit handled every 16-byte access separately and
//    was 72% busy) and stored row by row in LDS with an XOR swizzle of the
//    16-byte pieces that keeps both those writes and the fragment reads free
//    of bank conflicts.  The activation scales of the tile's rows, for all
//    K blocks, are copied to LDS once at its start with coalesced loads.
//  * Work order: all column tiles of one row tile are consecutive, so the
//    row tile's activations stay cached while the expert's weights stream.
//  * Row tiles come from a tile map built on the device from offsets, so no
//    count ever returns to the host.

#include "expert_gemm.h"
#include "moe_device.h"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// tiles[mt] = (expert, first row) for every tm-row tile of the padded
// expert segments, (-1, 0) for the unused entries up to mt_ub.  Offsets are
// clamped to the buffer so a corrupt plan cannot address past it.
__global__ __launch_bounds__(512) void gemm_tile_map_kernel(
    const int32_t* __restrict__ offsets, int E, int cap, int mt_ub, int tm,
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
      loc[i] = seg > 0 ? (seg + tm - 1) / tm : 0;
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
        tiles[start[e] + j] = make_int2(e, off[e] + j * tm);
}

// A workgroup computes a TMR (rows, 128 or 256) x 256 (columns) tile with 8
// waves (two per SIMD); wave (wm, wn) owns rows TMR/2 wm .. +TMR/2 and
// columns 64 wn .. +64, i.e. TMR/32 x 4 MFMA tiles.  Per 128-wide block each
// wave loads TMR/128 row groups of the activation tile and two of the
// weight tile (16 rows x 128 bytes each) into registers two blocks ahead and
// writes them to LDS one block ahead (two LDS stages), swizzled so that
// every ds_write_b128 and ds_read_b128 is conflict-free.  The activation
// scales of the tile's rows, all blocks, are copied to LDS once at the start
// (one scattered 4-byte load per row and block measured slower).  Per
// activation fragment, 4 MFMAs are issued back to back into separate result
// registers and then scaled into the fp32 accumulators, so one wave's
// scaling runs while the other wave's MFMAs occupy the matrix core.  A tile
// whose second row half lies past its segment skips that half's copies and
// MFMAs.
constexpr int kTN = 256;
template <int TMR> struct GemmTile {
  static constexpr int A = TMR * 128, B = kTN * 128;
  static constexpr int Stage = A + B;
  static constexpr int MI = TMR / 32;               // row fragments per wave
  static constexpr int AG = TMR / 128;              // row groups copied per wave
};

template <int YT, int TMR>
__global__ __launch_bounds__(512, 1) void expert_gemm_fp8_kernel(
    const unsigned char* __restrict__ rows, const float* __restrict__ rscale,
    int K, int cap, const int32_t* __restrict__ row_src,
    const int32_t* __restrict__ offsets, const unsigned char* __restrict__ w,
    const float* __restrict__ wscale, int N, unsigned char* __restrict__ y,
    const int2* __restrict__ tiles, int mt_ub, int ntn, int gn) {
  using G = GemmTile<TMR>;
  // one LDS object per stage, so the compiler can tell the block being read
  // from the block being written
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[G::Stage];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[G::Stage];
  __shared__ float sw[2][kGemmMaxK / 128];
  // the tile's activation scales, all blocks (row stride padded by one float
  // so the 16 rows of a fragment read distinct banks)
  constexpr int kRS = kGemmMaxK / 128 + 1;
  __shared__ float rsc[TMR * kRS];
  const int bid = blockIdx.x;
  const int ng = bid / (mt_ub * gn);
  const int rem = bid - ng * mt_ub * gn;
  const int mt = rem / gn;
  const int nt = ng * gn + (rem - mt * gn);
  if (mt >= mt_ub || nt >= ntn) return;
  const int2 tile = tiles[mt];
  const int e = tile.x;
  if (e < 0) return;
  const int r0 = tile.y;
  int r_end = offsets[e + 1];
  r_end = r_end > cap ? cap : r_end;
  r_end = r_end < r0 + TMR ? r_end : r0 + TMR;
  if (r_end <= r0) return;
  const int KB = K / 128;
  const int NB = N / 128;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int wm = wv & 1, wn = wv >> 1;
  // this wave's row half holds rows of the segment (uniform per wave)
  const bool half_live = (TMR / 2) * wm < r_end - r0;

  // weight scales of the tile's two 128-column blocks, and the activation
  // scales of its rows (one coalesced copy of TMR * KB consecutive floats;
  // rows past the segment repeat its last row and are never stored)
  for (int i = tid; i < 2 * KB; i += 512) {
    const int h = i / KB, b = i - h * KB;
    const int nb = nt * 2 + h < NB ? nt * 2 + h : NB - 1;
    sw[h][b] = wscale[((size_t)e * NB + nb) * KB + b];
  }
  for (int i = tid; i < TMR * KB; i += 512) {
    const int rr = i / KB, b = i - rr * KB;
    const int r = r0 + rr < r_end ? r0 + rr : r_end - 1;
    rsc[rr * kRS + b] = rscale[(size_t)r * KB + b];
  }

  // Copies are coalesced: a 16-row x 128-byte group is two loads of 8 rows,
  // 8 lanes per row reading its 128 bytes (piece p = lane & 7).  In LDS a
  // group keeps its rows in order, 128 bytes each, with 16-byte piece p of
  // row r at slot p ^ swz(r); the fragment of lane (g, c) is pieces 2g and
  // 2g + 1 of row c.  This swizzle keeps both the 16-byte writes (8 lanes
  // per row) and the fragment reads (16 lanes, 16 rows) free of LDS bank
  // conflicts on gfx950 (a fragment-order layout measured 2-way conflicts on
  // its writes, half of the kernel's LDS cycles).
  auto row_ofs = [](int r, int p) {                  // byte offset in a group
    return r * 128 + ((p ^ ((r & 7) ^ ((r >> 3) & 1))) * 16);
  };
  const int lp = lane & 7, lr = lane >> 3;
  int wofs[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) wofs[u] = row_ofs(8 * u + lr, lp);
  const int rofs0 = row_ofs(c16, 2 * g4), rofs1 = row_ofs(c16, 2 * g4 + 1);
  // this lane's sources (block 0) as 32-bit byte offsets from uniform
  // bases (cap * K and N * K fit in 32 bits); block b adds b * 128
  const unsigned char* wexp = w + (size_t)e * N * K;
  uint32_t aoff[G::AG][2];
  bool aload[G::AG];
#pragma unroll
  for (int q = 0; q < G::AG; ++q) {
    const int grp = G::AG * wv + q;
    aload[q] = 16 * grp < r_end - r0;          // row group holds segment rows
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int r = r0 + 16 * grp + 8 * u + lr;
      r = r < r_end ? r : r_end - 1;
      aoff[q][u] = (uint32_t)r * (uint32_t)K + 16 * lp;
    }
  }
  uint32_t boff[2][2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int n = nt * kTN + 16 * (2 * wv + q) + 8 * u + lr;
      n = n < N ? n : N - 1;
      boff[q][u] = (uint32_t)n * (uint32_t)K + 16 * lp;
    }

  f32x4 acc[G::MI][4];
#pragma unroll
  for (int i = 0; i < G::MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // staging through registers: block b + 1 is loaded during block b - 1 and
  // written to LDS at the start of block b
  u32x4 ra_[G::AG][2], rb_[2][2];
  auto load_regs = [&](int b) {
    const size_t o = (size_t)b * 128;
#pragma unroll
    for (int q = 0; q < G::AG; ++q)
      if (aload[q]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) ra_[q][u] = ld16(rows + aoff[q][u] + o);
      }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int u = 0; u < 2; ++u) rb_[q][u] = ld16(wexp + boff[q][u] + o);
  };
  auto store_regs = [&](unsigned char* base) {
#pragma unroll
    for (int q = 0; q < G::AG; ++q)
      if (aload[q]) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
          *reinterpret_cast<u32x4*>(base + (G::AG * wv + q) * 2048 + wofs[u]) =
              ra_[q][u];
      }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        *reinterpret_cast<u32x4*>(base + G::A + (2 * wv + q) * 2048 +
                                  wofs[u]) = rb_[q][u];
  };

  auto block = [&](int b, const unsigned char* base, unsigned char* next1) {
    __builtin_amdgcn_sched_barrier(0);   // keep blocks apart
    // unconditional (clamped) copies keep the compiler's wait counts
    // exact; past the last block they are redundant and never read
    lds_barrier();
    store_regs(next1);
    load_regs(b + 2 < KB ? b + 2 : KB - 1);
    if (!half_live) return;
    const float* sa = rsc + ((TMR / 2) * wm) * kRS + b;
    const float swb = sw[wn >> 1][b];
    i32x8 fb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned char* pb = base + G::A + (4 * wn + j) * 2048;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(pb + rofs0);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(pb + rofs1);
      fb[j] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                    (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int i = 0; i < G::MI; ++i) {
      const unsigned char* pa = base + (G::MI * wm + i) * 2048;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(pa + rofs0);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(pa + rofs1);
      const i32x8 fa = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                             (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const float si = sa[(16 * i + c16) * kRS] * swb;
      f32x4 p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        p[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            fb[j], fa, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(p[j][q], si, acc[i][j][q]);
    }
  };
  load_regs(0);
  store_regs(lds0);
  load_regs(KB > 1 ? 1 : 0);
  __syncthreads();   // sw (and block 0) visible
  // block b reads stage b % 2; two blocks per iteration with no branch
  // between them (exact wait counts), then the last one
  int b = 0;
  for (; b + 2 <= KB; b += 2) {
    block(b, lds0, lds1);
    block(b + 1, lds1, lds0);
  }
  if (b < KB) block(b, lds0, lds1);

  // lane: row TMR/2 wm + 16 i + c16, columns 64 wn + 16 j + 4 g4 .. + 3
  if (!half_live) return;
#pragma unroll
  for (int i = 0; i < G::MI; ++i) {
    const int r = r0 + (TMR / 2) * wm + 16 * i + c16;
    if (r >= r_end) continue;
    const bool live = row_src == nullptr || row_src[r] >= 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = nt * kTN + 64 * wn + 16 * j + 4 * g4;
      if (n >= N) continue;
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
  constexpr int TMR = kGemmRowsPerTile;
  const long long mt_ub = gemm_row_tiles(rows_capacity, E);
  int2* tiles = (int2*)workspace;
  const int cap = (int)rows_capacity;
  hipLaunchKernelGGL(gemm_tile_map_kernel, dim3(1), dim3(512), 0, s, offsets,
                     E, cap, (int)mt_ub, TMR, tiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // all column tiles of a row tile are consecutive: the row tile's
  // activations stay in cache while the expert's weight panels stream
  const int ntn = (N + kTN - 1) / kTN;
  const int gn = ntn;
  const long long grid = mt_ub * gn;
  const unsigned char* rb = (const unsigned char*)rows;
  const unsigned char* wb = (const unsigned char*)w;
  unsigned char* yb = (unsigned char*)y;
  if (y_dtype == MOE_BF16)
    hipLaunchKernelGGL((expert_gemm_fp8_kernel<1, TMR>), dim3((unsigned)grid),
                       dim3(512), 0, s, rb, row_scales, K, cap, row_src,
                       offsets, wb, w_scales, N, yb, tiles, (int)mt_ub, ntn,
                       gn);
  else
    hipLaunchKernelGGL((expert_gemm_fp8_kernel<0, TMR>), dim3((unsigned)grid),
                       dim3(512), 0, s, rb, row_scales, K, cap, row_src,
                       offsets, wb, w_scales, N, yb, tiles, (int)mt_ub, ntn,
                       gn);
  return hipGetLastError();
}

}  // namespace moe
