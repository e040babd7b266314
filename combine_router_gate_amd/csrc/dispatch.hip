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
  const int nte = ((T + 63) / 64) * E;
  unsigned long long* bits = plan_lds;
  int* base = reinterpret_cast<int*>(bits + nte);
  int* cnt = base + nte;
  int* off = cnt + E;
  local_plan(topk_idx, T, k, E, pad, bits, base, cnt, off);
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
      if (e < E) counts[e] = cnt[e];
      offsets[e] = off[e];
    }
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if ((int)blockIdx.x >= tok_blocks) {
    fill_padding_rows(blockIdx.x - tok_blocks, kDispatchFillBlocks, E, cnt,
                      off, capacity, row_src);
    return;
  }
  const int gw = blockIdx.x * 4 + wv;
  const int t = gw / hsplit, part = gw - t * hsplit;
  if (t >= T) return;
  int r = -1;
  if (lane < k) {
    const int e = topk_idx[(size_t)t * k + lane];
    if (e >= 0 && e < E) {
      const int q = (t >> 6) * E + e;
      r = base[q] + __popcll(bits[q] & ((1ull << (t & 63)) - 1ull));
      if ((long long)r >= capacity) r = -1;
    }
  }
  int rj[KMAX];
  publish_rows<KMAX>(r, t, part, lane, k, row_src, tok_row, rj);
  scatter_token_part<KMAX, MODE, U>(x, esize, H, t, part, hsplit, lane, rj,
                                    rows, row_scales);
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

// Scatter geometry: every group of u 64-lane chunks of a token row is a wave
// of its own (a token's waves run side by side); u = 1 when groups of two
// chunks would leave fewer than 16384 waves (Mixtral 4096 tokens: 26 -> 22
// us, MoonEP 8192 tokens of 768: 26.4 -> 24.5 us) or a half-empty last group
// (DeepSeek-V3 fp8 rows of 448 chunks: 204 -> 202 us).
struct ScatterShape {
  int mode, esize, u, hs, tblocks;
};
static ScatterShape scatter_shape(int xdt, int pdt, int T, int H,
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
