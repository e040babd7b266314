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
//  * A workgroup computes a 256x256 tile with 8 waves (two per SIMD, 128x64
//    each: 12 fragments read from LDS per 32 MFMAs, accumulators in 128
//    VGPRs).  Operands reach LDS through direct global->LDS copies into two
//    stages (no staging registers, which is what lets the 256-row tile fit),
//    stored row by row with an XOR swizzle of the 16-byte pieces that keeps
//    the fragment reads free of bank conflicts; the activation scales of a
//    block travel with it.
//  * Each wave's block is software-pipelined: the next activation fragment
//    is read while the current MFMAs run, and their products are scaled
//    into the accumulators during the next step, under a raised wave
//    priority so the two waves of a SIMD drift apart and one's LDS reads
//    overlap the other's MFMAs.
//  * Work order: workgroups land on the 8 XCDs round-robin; column tiles are
//    placed so each one stays on one XCD for every row tile, so an expert's
//    weight panels are read into one L2 while its activation rows are
//    shared across XCDs.
//  * Row tiles come from a tile map built on the device from offsets, so no
//    count ever returns to the host.

#include "expert_gemm.h"
#include "moe_device.h"
#include "moe_scan.h"

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
  for (int e = tid; e < E; e += 512) {
    const int seg = off[e + 1] - off[e];
    start[e] = seg > 0 ? (seg + tm - 1) / tm : 0;
  }
  __syncthreads();
  if (tid < 64) {
    const int total =
        wave_exclusive_scan<MOE_MAX_EXPERTS / 64>(start, E, nullptr);
    if (tid == 0) start[E] = total;
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

// A workgroup computes a 256 (rows) x 256 (columns) tile with 8 waves (two
// per SIMD); wave (wm, wn) owns rows 128 wm .. +128 and columns 64 wn .. +64,
// i.e. 8 x 4 MFMA tiles: 12 fragments read from LDS per 32 MFMAs.  Operands
// reach LDS through direct global->LDS copies, two stages: while block b is
// computed from one stage, block b + 1 is copied into the other, and one
// wait plus barrier per block hands the stages over.  Each wave copies 32
// activation rows and 32 weight rows (16 rows x 128 bytes per group) and the
// activation scales of its rows for that block.  Rows sit in LDS with an XOR
// swizzle of their 16-byte pieces that keeps the fragment reads free of bank
// conflicts.
//
// The block's work is software-pipelined per wave: the activation fragment
// of step i + 1 is read while the 4 MFMAs of step i run, and the products of
// step i are scaled into the fp32 accumulators during step i + 1 (those of
// the block's last step during the next block's first), so neither the LDS
// latency nor the MFMA latency sits between dependent instructions.  Right
// after the barrier the next block's weight fragments and first activation
// fragment are read while the last MFMAs drain.  A tile whose second row
// half lies past its segment skips that half's fragment reads and MFMAs.
constexpr int kTM = 256, kTN = 256;
constexpr int kStageA = kTM * 128, kStageB = kTN * 128;
constexpr int kStage = kStageA + kStageB;   // 64 KiB
constexpr int kMI = 8;                      // row fragments per wave

// Work order: the hardware places workgroup ids round-robin over the 8
// XCDs (id % 8), each with its own L2.  Row tiles go in groups of G =
// 8 / gcd(ntn, 8), so that a group holds a multiple of 8 workgroups, and
// inside a group column tiles go in chunks of 8, each chunk holding its 8
// columns for every row tile of the group.  Column tile nt then runs on XCD
// nt % 8 for every row tile (the last ntn % 8 columns excepted), so all row
// tiles of an expert find its weight panels in one L2, while a row tile's
// activation panel is shared by the column tiles on every XCD.
__device__ __forceinline__ int row_group(int ntn) {
  const int g = ntn & 7;   // gcd(ntn, 8) is 8, 4, 2 or 1
  return g == 0 ? 1 : (g & 3) == 0 ? 2 : (g & 1) == 0 ? 4 : 8;
}
__device__ __forceinline__ void tile_of(int bid, int ntn, int* mt, int* nt) {
  const int G = row_group(ntn);
  const int grp = bid / (G * ntn);
  const int rem = bid - grp * G * ntn;
  const int full = (ntn / 8) * 8 * G;
  if (rem < full) {
    const int chunk = rem / (8 * G), within = rem - chunk * 8 * G;
    *mt = G * grp + within / 8;
    *nt = 8 * chunk + (within & 7);
  } else {
    const int tail = ntn & 7;
    *mt = G * grp + (rem - full) / tail;
    *nt = (ntn / 8) * 8 + (rem - full) % tail;
  }
}

template <int YT>
__global__ __launch_bounds__(512, 1) void expert_gemm_fp8_kernel(
    const unsigned char* __restrict__ rows, const float* __restrict__ rscale,
    int K, int cap, const int32_t* __restrict__ row_src,
    const int32_t* __restrict__ offsets, const unsigned char* __restrict__ w,
    const float* __restrict__ wscale, int N, unsigned char* __restrict__ y,
    const int2* __restrict__ tiles, int mt_ub, int ntn) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[kStage];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[kStage];
  __shared__ float sw[2][kGemmMaxK / 128];
  // activation scales of the stage's block: wave v copies rows 32 v .. +31
  // (lanes 32..63 repeat them) to rsr[stage][64 v .. 64 v + 63]
  __shared__ __attribute__((aligned(256))) float rsr[2][8 * 64];
  int mt, nt;
  tile_of(blockIdx.x, ntn, &mt, &nt);
  if (mt >= mt_ub || nt >= ntn) return;
  const int2 tile = tiles[mt];
  const int e = tile.x;
  if (e < 0) return;
  const int r0 = tile.y;
  int r_end = offsets[e + 1];
  r_end = r_end > cap ? cap : r_end;
  r_end = r_end < r0 + kTM ? r_end : r0 + kTM;
  if (r_end <= r0) return;
  const int KB = K / 128;
  const int NB = N / 128;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int wm = wv & 1, wn = wv >> 1;
  // this wave's row half holds rows of the segment (uniform per wave)
  const bool half_live = 128 * wm < r_end - r0;

  // weight scales of the tile's two 128-column blocks
  for (int i = tid; i < 2 * KB; i += 512) {
    const int h = i / KB, b = i - h * KB;
    const int nb = nt * 2 + h < NB ? nt * 2 + h : NB - 1;
    sw[h][b] = wscale[((size_t)e * NB + nb) * KB + b];
  }

  // A 16-row x 128-byte group is two copies of 8 rows, 8 lanes per row.  In
  // LDS a group keeps its rows in order, 128 bytes each, with 16-byte piece
  // p of row r at slot p ^ swz(r); a copy writes lane l at slot l & 7 of row
  // l >> 3, so lane l reads piece (l & 7) ^ swz(row) of its row.  The
  // fragment of lane (g, c) is pieces 2g and 2g + 1 of row c.  The swizzle
  // keeps the fragment reads (16 lanes, 16 rows) free of bank conflicts.
  auto swz = [](int r) { return (r & 7) ^ ((r >> 3) & 1); };
  auto row_ofs = [&](int r, int p) { return r * 128 + ((p ^ swz(r)) * 16); };
  const int lp = lane & 7, lr = lane >> 3;
  const int rofs0 = row_ofs(c16, 2 * g4), rofs1 = row_ofs(c16, 2 * g4 + 1);
  // this lane's sources (block 0) as 32-bit byte offsets from uniform bases
  // (cap * K and N * K fit in 32 bits); block b moves the bases by b * 128.
  // Rows past the segment repeat its last row (copied, never stored).
  const unsigned char* wexp = w + (size_t)e * N * K;
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int r = r0 + 32 * wv + 16 * h + 8 * u + lr;
      r = r < r_end ? r : r_end - 1;
      aoff[2 * h + u] = (uint32_t)r * (uint32_t)K + 16 * (lp ^ swz(8 * u + lr));
      int n = nt * kTN + 32 * wv + 16 * h + 8 * u + lr;
      n = n < N ? n : N - 1;
      boff[2 * h + u] = (uint32_t)n * (uint32_t)K + 16 * (lp ^ swz(8 * u + lr));
    }
  int sr = r0 + 32 * wv + (lane & 31);
  sr = sr < r_end ? sr : r_end - 1;
  const uint32_t soff = (uint32_t)sr * (uint32_t)KB * 4u;

  // the 9 copies of block b into one stage (same count for every wave)
  auto copy_block = [&](int b, unsigned char* stage, float* scales) {
    const uint32_t o = (uint32_t)b * 128u;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      copy_to_lds16(rows + o, aoff[q],
                    lds_addr(stage + (2 * wv + (q >> 1)) * 2048 + (q & 1) * 1024));
#pragma unroll
    for (int q = 0; q < 4; ++q)
      copy_to_lds16(wexp + o, boff[q],
                    lds_addr(stage + kStageA + (2 * wv + (q >> 1)) * 2048 +
                             (q & 1) * 1024));
    copy_to_lds4(rscale + b, soff, lds_addr(scales + 64 * wv));
  };

  f32x4 acc[kMI][4];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto read_frag = [&](const unsigned char* p) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(p + rofs0);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(p + rofs1);
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  // scale of row 128 wm + 16 i + c16, copied by wave 4 wm + i / 2
  auto row_scale = [&](const float* scales, int i) {
    return scales[(4 * wm + i / 2) * 64 + 16 * (i & 1) + c16];
  };
  i32x8 fb[4], fa;
  f32x4 pp[4];        // products of the previous step, not yet scaled
  float sp = 0.f;     // their scale
  auto load_block = [&](const unsigned char* base) {
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = read_frag(base + kStageA + (4 * wn + j) * 2048);
    fa = read_frag(base + (kMI * wm) * 2048);
  };
  auto retire = [&](int i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(pp[j][q], sp, acc[i][j][q]);
  };
  // block b from stage `base`; fb and fa of step 0 are already loaded
  auto compute = [&](int b, const unsigned char* base, const float* scales) {
    const float swb = sw[wn >> 1][b];
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
      i32x8 fn;
      if (i + 1 < kMI) fn = read_frag(base + (kMI * wm + i + 1) * 2048);
      const float si = row_scale(scales, i) * swb;
      f32x4 p[4];
      // raised wave priority while this step's MFMAs and the previous
      // step's scale-FMAs issue: the two waves of a SIMD, released together
      // by each barrier, then drift apart so one's LDS reads overlap the
      // other's MFMAs (measured 5-9 % faster, same bits)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        p[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            fb[j], fa, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
      if (i > 0) retire(i - 1);
      else if (b > 0) retire(kMI - 1);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) pp[j] = p[j];
      sp = si;
      if (i + 1 < kMI) fa = fn;
    }
  };
  // block b: copy block b + 1 into the stage block b - 1 used, compute block
  // b, wait for this wave's copies and meet the other waves (stage b + 1 is
  // complete and nobody reads stage b any more), then read block b + 1's
  // first fragments
  auto step = [&](int b, const unsigned char* cur, const float* cur_s,
                  unsigned char* nxt, float* nxt_s) {
    __builtin_amdgcn_sched_barrier(0);
    if (b + 1 < KB) copy_block(b + 1, nxt, nxt_s);
    if (half_live) compute(b, cur, cur_s);
    copies_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (half_live && b + 1 < KB) load_block(nxt);
  };
  __syncthreads();   // sw visible; no load of this wave in flight
  copy_block(0, lds0, rsr[0]);
  copies_barrier();
  if (half_live) load_block(lds0);
  int b = 0;
  for (; b + 2 <= KB; b += 2) {
    step(b, lds0, rsr[0], lds1, rsr[1]);
    step(b + 1, lds1, rsr[1], lds0, rsr[0]);
  }
  if (b < KB) step(b, lds0, rsr[0], lds1, rsr[1]);
  if (!half_live) return;   // no copy in flight: every step waited for them
  retire(kMI - 1);

  // lane: row 128 wm + 16 i + c16, columns 64 wn + 16 j + 4 g4 .. + 3
#pragma unroll
  for (int i = 0; i < kMI; ++i) {
    const int r = r0 + 128 * wm + 16 * i + c16;
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
  const long long mt_ub = gemm_row_tiles(rows_capacity, E);
  int2* tiles = (int2*)workspace;
  const int cap = (int)rows_capacity;
  hipLaunchKernelGGL(gemm_tile_map_kernel, dim3(1), dim3(512), 0, s, offsets,
                     E, cap, (int)mt_ub, kTM, tiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int ntn = (N + kTN - 1) / kTN;
  // row tiles in groups of G (tile_of), every column tile of each
  const int G = (ntn & 7) == 0 ? 1 : (ntn & 3) == 0 ? 2 : (ntn & 1) == 0 ? 4 : 8;
  const long long grid = (mt_ub + G - 1) / G * G * ntn;
  const unsigned char* rb = (const unsigned char*)rows;
  const unsigned char* wb = (const unsigned char*)w;
  unsigned char* yb = (unsigned char*)y;
  if (y_dtype == MOE_BF16)
    hipLaunchKernelGGL(expert_gemm_fp8_kernel<1>, dim3((unsigned)grid),
                       dim3(512), 0, s, rb, row_scales, K, cap, row_src,
                       offsets, wb, w_scales, N, yb, tiles, (int)mt_ub, ntn);
  else
    hipLaunchKernelGGL(expert_gemm_fp8_kernel<0>, dim3((unsigned)grid),
                       dim3(512), 0, s, rb, row_scales, K, cap, row_src,
                       offsets, wb, w_scales, N, yb, tiles, (int)mt_ub, ntn);
  return hipGetLastError();
}

}  // namespace moe
