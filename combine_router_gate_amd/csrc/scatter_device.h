// Device code of the scatter shared by dispatch.hip and the one-launch
// route + dispatch of route.hip: destination rows, padding fill, the row
// copy (optionally quantised to fp8 E4M3 with 1x128 scales), the small-batch
// plan rebuilt in LDS, and the scatter geometry.
#pragma once

#include "moe_device.h"
#include "moe_scan.h"
#include "moe_launch.h"

namespace moe {

constexpr int kDispatchFillBlocks = 64;

// Resolve the k destination rows of token t; lanes >= k hold -1.  A row
// outside [0, capacity) -- possible only if counts/offsets/workspace come
// from different calls -- is dropped rather than written.
__device__ __forceinline__ int token_row(
    int t, int lane, int k, int E, long long capacity,
    const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ tile_base,
    const int32_t* __restrict__ slot_rank) {
  int r = -1;
  if (lane < k) {
    const size_t s = (size_t)t * k + lane;
    const int e = topk_idx[s];
    if (e >= 0 && e < E) {
      const int rank = slot_rank[s];
      r = tile_base[(size_t)(t / kTileT) * E + e] + rank;
      if (rank < 0 || r < 0 || (long long)r >= capacity) r = -1;
    }
  }
  return r;
}

// Rows past every expert's tokens: row_src = -1 for the padding rows of each
// expert and every row from offsets[E] to capacity; fill block fb of nfb.
__device__ __forceinline__ void fill_padding_rows(
    int fb, int nfb, int E, const int32_t* counts, const int32_t* offsets,
    long long capacity, int32_t* __restrict__ row_src) {
  for (int e = fb; e < E; e += nfb) {
    const long long hi = min((long long)offsets[e + 1], capacity);
    for (long long r = (long long)offsets[e] + counts[e] + threadIdx.x;
         r < hi; r += blockDim.x)
      if (r >= 0) row_src[r] = -1;
  }
  for (long long r = max((long long)offsets[E], 0LL) + (long long)fb *
                         blockDim.x + threadIdx.x;
       r < capacity; r += (long long)nfb * blockDim.x)
    row_src[r] = -1;
}

// MODE 0: exact copy (x and payload of the same 2- or 4-byte type)
// MODE 1: bf16 x -> fp8;  MODE 2: fp32 x -> fp8
// U: 64-lane chunks per lane step (2 keeps two loads in flight per lane; 1
// lets few tokens spread over twice as many waves)
// One wave's share (part of hsplit) of token t's row, copied or quantised to
// every destination row rj[j] >= 0.
template <int KMAX, int MODE, int U>
__device__ __forceinline__ void scatter_token_part(
    const unsigned char* __restrict__ x, int esize, int H, int t, int part,
    int hsplit, int lane, const int (&rj)[KMAX],
    unsigned char* __restrict__ rows, float* __restrict__ row_scales) {
  if constexpr (MODE == 0) {
    const size_t rowb = (size_t)H * esize;
    const int nc = (int)(rowb / 16);
    const unsigned char* src = x + (size_t)t * rowb;
    for (int c0 = part * 64 * U; c0 < nc; c0 += hsplit * 64 * U) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < nc) v[u] = ld16_stream(src + (size_t)c * 16);
      }
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (rj[j] < 0) continue;
        unsigned char* dst = rows + (size_t)rj[j] * rowb;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * 64 + lane;
          if (c < nc) st16_stream(dst + (size_t)c * 16, v[u]);
        }
      }
    }
  } else {
    // 16 consecutive elements per lane; 8 lanes per 128-element block; U
    // 64-lane chunks per iteration, all loaded before any is used, with
    // loads clamped to the row (never conditional) so they stay in flight
    // together
    constexpr int EB = MODE == 1 ? 32 : 64;    // source bytes per lane chunk
    const int nc16 = H / 16;
    const int nblk = H / kFp8Block;
    const unsigned char* src = x + (size_t)t * H * esize;
    for (int c0 = part * 64 * U; c0 < nc16; c0 += hsplit * 64 * U) {
      u32x4 v[U][EB / 16];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * 64 + lane;
        const unsigned char* p = src + (size_t)(c < nc16 ? c : nc16 - 1) * EB;
#pragma unroll
        for (int q = 0; q < EB / 16; ++q) v[u][q] = ld16_stream(p + 16 * q);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * 64 + lane;
        float f[16];
        if constexpr (MODE == 1) {
          unpack8_bf16(v[u][0], f);
          unpack8_bf16(v[u][1], f + 8);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) f[4 * q + i] = __uint_as_float(v[u][q][i]);
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
        for (int m = 4; m >= 1; m >>= 1)
          amax = fmaxf(amax, __shfl_xor(amax, m, 8));
        // scale and quotient are IEEE fp32 operations (correctly rounded)
        const float s = amax > 0.0f ? amax / kFp8Max : 1.0f;
        float q[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = f[i] / s;
        u32x4 pk;
        pk.x = e4m3_encode4(q[0], q[1], q[2], q[3]);
        pk.y = e4m3_encode4(q[4], q[5], q[6], q[7]);
        pk.z = e4m3_encode4(q[8], q[9], q[10], q[11]);
        pk.w = e4m3_encode4(q[12], q[13], q[14], q[15]);
        if (c < nc16) {
#pragma unroll
          for (int j = 0; j < KMAX; ++j) {
            if (rj[j] < 0) continue;
            st16_stream(rows + (size_t)rj[j] * H + (size_t)c * 16, pk);
            if ((lane & 7) == 0) row_scales[(size_t)rj[j] * nblk + c / 8] = s;
          }
        }
      }
    }
  }
}

// Lane j < k holds row r of slot (t, j): record it (part 0 only) and
// broadcast all k rows to every lane.
template <int KMAX>
__device__ __forceinline__ void publish_rows(int r, int t, int part, int lane,
                                             int k, int32_t* __restrict__ row_src,
                                             int32_t* __restrict__ tok_row,
                                             int (&rj)[KMAX]) {
  if (lane < k && part == 0) {
    tok_row[(size_t)t * k + lane] = r;
    if (r >= 0) row_src[r] = t;
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    rj[j] = (j < k) ? __builtin_amdgcn_readlane(r, j) : -1;
}

// ------------------------------------------------------------------ small batches

// The routing plan of T <= kSmallPlanT tokens rebuilt in one workgroup's LDS
// (the same results as the plan kernels): a ballot per (64-token tile,
// expert) set by LDS atomics, counts by popcount, the exclusive scan of the
// padded counts, and the first row of every (tile, expert).
__device__ void local_plan(const int32_t* __restrict__ topk_idx, int T, int k,
                           int E, int pad, unsigned long long* bits, int* base,
                           int* cnt, int* off) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int nt = (T + 63) / 64;
  for (int i = tid; i < nt * E; i += nthr) bits[i] = 0ull;
  __syncthreads();
  for (int p = tid; p < T * k; p += nthr) {
    const int e = topk_idx[p];
    const int t = p / k;
    if (e >= 0 && e < E) atomicOr(&bits[(t >> 6) * E + e], 1ull << (t & 63));
  }
  __syncthreads();
  for (int e = tid; e < E; e += nthr) {
    int c = 0;
    for (int q = 0; q < nt; ++q) c += __popcll(bits[q * E + e]);
    cnt[e] = c;
    off[e] = (c + pad - 1) / pad * pad;
  }
  __syncthreads();
  if (tid < 64) {
    // exclusive scan of the padded counts
    const int total =
        wave_exclusive_scan<MOE_MAX_EXPERTS / 64>(off, E, nullptr);
    if (tid == 0) off[E] = total;
  }
  __syncthreads();
  for (int e = tid; e < E; e += nthr) {
    int run = off[e];
    for (int q = 0; q < nt; ++q) {
      base[q * E + e] = run;
      run += __popcll(bits[q * E + e]);
    }
  }
  __syncthreads();
}

inline size_t local_plan_lds_bytes(int T, int E) {
  const size_t nte = (size_t)((T + 63) / 64) * E;
  return nte * 8 + nte * 4 + (size_t)E * 4 + (size_t)(E + 1) * 4;
}

// LDS arrays of local_plan for T tokens and E experts (bits, then first rows,
// counts, offsets), carved from one dynamic LDS block.
struct LocalPlan {
  unsigned long long* bits;
  int *base, *cnt, *off;
};
__device__ __forceinline__ LocalPlan local_plan_arrays(unsigned long long* lds,
                                                       int T, int E) {
  const int nte = ((T + 63) / 64) * E;
  LocalPlan p;
  p.bits = lds;
  p.base = reinterpret_cast<int*>(lds + nte);
  p.cnt = p.base + nte;
  p.off = p.cnt + E;
  return p;
}

// Block blk of the small-batch scatter once the plan p is in LDS: block 0
// also stores counts and offsets; blocks from tok_blocks on fill padding
// rows, the others scatter their waves' (token, part) pairs.
template <int KMAX, int MODE, int U>
__device__ __forceinline__ void plan_dispatch_block(
    int blk, const unsigned char* __restrict__ x, int esize, int T, int H,
    const int32_t* __restrict__ topk_idx, int k, int E,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    unsigned char* __restrict__ rows, long long capacity,
    float* __restrict__ row_scales, int32_t* __restrict__ row_src,
    int32_t* __restrict__ tok_row, int tok_blocks, int hsplit,
    const LocalPlan& p) {
  if (blk == 0) {
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
      if (e < E) counts[e] = p.cnt[e];
      offsets[e] = p.off[e];
    }
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (blk >= tok_blocks) {
    fill_padding_rows(blk - tok_blocks, kDispatchFillBlocks, E, p.cnt,
                      p.off, capacity, row_src);
    return;
  }
  const int gw = blk * 4 + wv;
  const int t = gw / hsplit, part = gw - t * hsplit;
  if (t >= T) return;
  int r = -1;
  if (lane < k) {
    const int e = topk_idx[(size_t)t * k + lane];
    if (e >= 0 && e < E) {
      const int q = (t >> 6) * E + e;
      r = p.base[q] + __popcll(p.bits[q] & ((1ull << (t & 63)) - 1ull));
      if ((long long)r >= capacity) r = -1;
    }
  }
  int rj[KMAX];
  publish_rows<KMAX>(r, t, part, lane, k, row_src, tok_row, rj);
  scatter_token_part<KMAX, MODE, U>(x, esize, H, t, part, hsplit, lane, rj,
                                    rows, row_scales);
}

// Scatter geometry: every group of u 64-lane chunks of a token row is a wave
// of its own (a token's waves run side by side); u = 1 when groups of two
// chunks would leave fewer than 16384 waves (Mixtral 4096 tokens: 26 -> 22
// us, MoonEP 8192 tokens of 768: 26.4 -> 24.5 us) or a half-empty last group
// (DeepSeek-V3 fp8 rows of 448 chunks: 204 -> 202 us).
struct ScatterShape {
  int mode, esize, u, hs, tblocks;
};
inline ScatterShape scatter_shape(int xdt, int pdt, int T, int H,
                                  bool allow_u2 = true) {
  ScatterShape g;
  g.esize = xdt == DT_F32 ? 4 : 2;
  g.mode = pdt != DT_FP8 ? 0 : (xdt == DT_BF16 ? 1 : 2);
  const int nch = g.mode == 0 ? H * g.esize / 16 : H / 16;  // lane chunks
  g.u = allow_u2 && (long long)T * ((nch + 127) / 128) >= 16384 &&
                nch % 128 == 0
            ? 2
            : 1;
  g.hs = (nch + 64 * g.u - 1) / (64 * g.u);
  g.hs = g.hs < 1 ? 1 : g.hs;
  g.tblocks = (int)(((long long)T * g.hs + 3) / 4);
  return g;
}

}  // namespace moe
