// Router gate (MFMA), softmax top-k with renormalised weights, per-expert
// tile histogram and padded exclusive scan for gfx950.
//
// The router is a small linear layer whose softmax gives a probability
// distribution over the experts; the top-k experts are kept and their
// outputs later weighted by that distribution ("Efficient and Portable
// Mixture-of-Experts Communication", Introduction).  Token counts per
// destination expert are the first thing that page's dispatch computes
// (section Dispatch); segments are padded per expert and exclusively scanned
// into MoonEP-style `cu_seqlens` ("MoonEP developer guide", core API example,
// `token_padding`).
//
// Design for CDNA4:
//  * Gate GEMM l = x W^T on the matrix cores: v_mfma_f32_16x16x32_bf16 for
//    bf16 inputs, v_mfma_f32_16x16x4_f32 for fp32 inputs, fp32 accumulation.
//    A wave owns a 16-token x (16*ET)-expert block of logits in registers, so
//    softmax and top-k run on-chip and the logits never touch HBM.
//  * E >= 64: a workgroup of 4 waves covers 64 tokens and stages the gate
//    weight through LDS in 128-byte k-chunks shared by the 4 waves; x is
//    streamed once with non-temporal loads.
//  * E < 64 (memory-bound gate): the 4 waves split the hidden dimension of a
//    16-token tile and reduce their partial logits through LDS in a fixed
//    order, so four times as many workgroups stream x.
//  * Top-k: the 16 lanes of a lane group hold all logits of one token; k
//    rounds of a 16-lane max over 64-bit keys (order-preserving logit key,
//    then inverted expert id) give the lowest-index tie-break exactly.
//    Weights are exp(l_j - l_max) / sum over the chosen, i.e. the full
//    softmax renormalised over the chosen experts (the all-expert
//    denominator cancels).
//  * Histogram: per 64-token tile, an LDS bitmap per expert (bit = token)
//    assembled with ds_or_b64; its popcount is the tile count and the
//    popcount of the bits below a token is that token's rank, which fixes a
//    stable, deterministic slot order with no global atomics.
//  * Scan: one workgroup scans the [tiles, E] counts (chunked over tiles,
//    then an LDS scan over experts) and leaves, in place, the first row of
//    every (tile, expert) run.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

// ------------------------------------------------------------------ MFMA

// 8 consecutive k-elements of one row: the operand a lane contributes for
// one 32-wide k step.  All lanes and both operands use the same k order, so
// any assignment of the 32 k values to (lane group, element) is a valid
// reordering of the dot product.
template <typename XT> struct Frag;
template <> struct Frag<uint16_t> { u32x4 v; };          // 8 bf16
template <> struct Frag<float> { u32x4 v0, v1; };        // 8 fp32

template <typename XT>
__device__ __forceinline__ void frag_load(Frag<XT>& f, const XT* p, bool ok,
                                          bool stream);
template <>
__device__ __forceinline__ void frag_load<uint16_t>(Frag<uint16_t>& f,
                                                    const uint16_t* p, bool ok,
                                                    bool stream) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  f.v = ok ? (stream ? ld16_stream(p) : ld16(p)) : z;
}
template <>
__device__ __forceinline__ void frag_load<float>(Frag<float>& f,
                                                 const float* p, bool ok,
                                                 bool stream) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  f.v0 = ok ? (stream ? ld16_stream(p) : ld16(p)) : z;
  f.v1 = ok ? (stream ? ld16_stream(p + 4) : ld16(p + 4)) : z;
}

__device__ __forceinline__ f32x4 mfma_step(const Frag<uint16_t>& a,
                                           const Frag<uint16_t>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a.v), __builtin_bit_cast(bf16x8, b.v), c, 0,
      0, 0);
}
__device__ __forceinline__ f32x4 mfma_step(const Frag<float>& a,
                                           const Frag<float>& b, f32x4 c) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v0[s]),
                                             __uint_as_float(b.v0[s]), c, 0,
                                             0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v1[s]),
                                             __uint_as_float(b.v1[s]), c, 0,
                                             0, 0);
  return c;
}

// ------------------------------------------------------------------ top-k

// acc[et][i] holds the logit of token t0 + 4*(lane/16) + i and expert
// 16*et + lane%16 (the 16x16 MFMA output layout).
template <int ET>
__device__ __forceinline__ void topk_epilogue(
    const f32x4 (&acc)[ET], int t0, int T, int E, int k,
    const float* __restrict__ bias, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ logits_dbg) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  float bv[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et) {
    const int e = et * 16 + c;
    bv[et] = (bias != nullptr && e < E) ? bias[e] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + g * 4 + i;
    float v[ET];
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      v[et] = acc[et][i] + bv[et];
      const int e = et * 16 + c;
      if (logits_dbg != nullptr && t < T && e < E)
        logits_dbg[(size_t)t * E + e] = v[et];
    }
    uint32_t taken = 0;
    int sel_e[MOE_MAX_TOPK];
    float sel_v[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      sel_e[j] = 0;
      sel_v[j] = 0.0f;
      if (j < k) {
        unsigned long long best = 0ull;
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          const int e = et * 16 + c;
          const unsigned long long key =
              ((unsigned long long)f32_order_key(v[et]) << 32) |
              (unsigned long long)(0xffffffffu - (uint32_t)e);
          const bool ok = e < E && !((taken >> et) & 1u);
          best = (ok && key > best) ? key : best;
        }
        best = max16_u64(best);
        const int ew = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffull));
        if ((ew & 15) == c) taken |= 1u << (ew >> 4);
        sel_e[j] = ew;
        sel_v[j] = f32_from_order_key((uint32_t)(best >> 32));
      }
    }
    float ex[MOE_MAX_TOPK];
    float den = 0.0f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      ex[j] = (j < k) ? expf(sel_v[j] - sel_v[0]) : 0.0f;
      den += ex[j];
    }
    if (t < T) {
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        if (j < k && c == j) {
          topk_idx[(size_t)t * k + j] = sel_e[j];
          topk_w[(size_t)t * k + j] = ex[j] / den;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ gate, E >= 64

// One workgroup = 4 waves = 64 tokens; wave w owns tokens [t0 + 16w, +16)
// and all 16*ET experts.  The gate weight goes through LDS in chunks of 128
// bytes of k per expert row (64 bf16 or 32 fp32), rows padded by 16 bytes.
template <typename XT, int ET>
__global__ __launch_bounds__(256) void gate_topk_wide_kernel(
    const XT* __restrict__ x, const XT* __restrict__ w,
    const float* __restrict__ bias, int T, int H, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits_dbg) {
  constexpr int EP = ET * 16;
  constexpr int ELEM16 = 16 / sizeof(XT);         // elements per 16 bytes
  constexpr int KC = 128 / sizeof(XT);            // k elements per chunk
  constexpr int KSTEPS = KC / 32;                 // 32-wide MFMA k steps
  constexpr int ROWB = 144;                       // 128 + 16 pad bytes
  constexpr int PIECES = EP * 8 / 256;            // 16-byte pieces/thread
  __shared__ __align__(16) unsigned char wlds[EP * ROWB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4;
  const int t0 = blockIdx.x * 64 + wv * 16;
  const int arow = t0 + (lane & 15);
  const bool arow_ok = arow < T;
  const XT* xrow = x + (size_t)(arow_ok ? arow : 0) * H;

  f32x4 acc[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et) acc[et] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wreg[PIECES];
  Frag<XT> anext[KSTEPS];
  const int nchunks = (H + KC - 1) / KC;

  auto load_w = [&](int kc) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int p = tid + 256 * i;
      const int e = p >> 3, cc = p & 7;
      const int kk = kc + cc * ELEM16;
      const u32x4 z = {0u, 0u, 0u, 0u};
      wreg[i] = (e < E && kk < H) ? ld16(w + (size_t)e * H + kk) : z;
    }
  };
  auto load_a = [&](int kc) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int kk = kc + s * 32 + g * 8;
      frag_load<XT>(anext[s], xrow + kk, arow_ok && kk < H, true);
    }
  };

  load_w(0);
  load_a(0);
  for (int ch = 0; ch < nchunks; ++ch) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int p = tid + 256 * i;
      st16(wlds + (p >> 3) * ROWB + (p & 7) * 16, wreg[i]);
    }
    __syncthreads();
    Frag<XT> acur[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) acur[s] = anext[s];
    if (ch + 1 < nchunks) {
      load_w((ch + 1) * KC);
      load_a((ch + 1) * KC);
    }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        const unsigned char* bp =
            wlds + (et * 16 + (lane & 15)) * ROWB + (s * 32 + g * 8) * sizeof(XT);
        Frag<XT> b;
        if constexpr (sizeof(XT) == 2) {
          b.v = *reinterpret_cast<const u32x4*>(bp);
        } else {
          b.v0 = *reinterpret_cast<const u32x4*>(bp);
          b.v1 = *reinterpret_cast<const u32x4*>(bp + 16);
        }
        acc[et] = mfma_step(acur[s], b, acc[et]);
      }
    }
  }
  topk_epilogue<ET>(acc, t0, T, E, k, bias, topk_idx, topk_w, logits_dbg);
}

// ------------------------------------------------------------------ gate, E < 64

// One workgroup = 16 tokens; the 4 waves split the hidden dimension into
// 32-aligned quarters, read both operands straight from global memory (the
// gate weight is small and cache-resident) and reduce through LDS in wave
// order 0,1,2,3.
template <typename XT, int ET>
__global__ __launch_bounds__(256) void gate_topk_ksplit_kernel(
    const XT* __restrict__ x, const XT* __restrict__ w,
    const float* __restrict__ bias, int T, int H, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits_dbg) {
  constexpr int U = 4;  // k steps in flight per wave
  __shared__ f32x4 red[3][ET][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4;
  const int t0 = blockIdx.x * 16;
  const int arow = t0 + (lane & 15);
  const bool arow_ok = arow < T;
  const XT* xrow = x + (size_t)(arow_ok ? arow : 0) * H;
  const XT* wrow[ET];
  bool wrow_ok[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et) {
    const int e = et * 16 + (lane & 15);
    wrow_ok[et] = e < E;
    wrow[et] = w + (size_t)(e < E ? e : 0) * H;
  }
  const int quarter = ((H + 3) / 4 + 31) / 32 * 32;
  const int k_lo = wv * quarter;
  const int k_hi = min(H, k_lo + quarter);

  f32x4 acc[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et) acc[et] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = k_lo; k0 < k_hi; k0 += 32 * U) {
    Frag<XT> a[U];
    Frag<XT> b[U][ET];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k0 + u * 32 + g * 8;
      const bool kok = kk < k_hi;
      frag_load<XT>(a[u], xrow + kk, arow_ok && kok, true);
#pragma unroll
      for (int et = 0; et < ET; ++et)
        frag_load<XT>(b[u][et], wrow[et] + kk, wrow_ok[et] && kok, false);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int et = 0; et < ET; ++et) acc[et] = mfma_step(a[u], b[u][et], acc[et]);
  }
  if (wv > 0) {
#pragma unroll
    for (int et = 0; et < ET; ++et) red[wv - 1][et][lane] = acc[et];
  }
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int et = 0; et < ET; ++et) acc[et] += red[q][et][lane];
    topk_epilogue<ET>(acc, t0, T, E, k, bias, topk_idx, topk_w, logits_dbg);
  }
}

// ------------------------------------------------------------------ histogram

// One workgroup per 64-token tile.  bits[e] has bit i set iff token t0+i
// chose expert e: the tile's "ballot" for e, assembled in LDS.
__global__ __launch_bounds__(256) void tile_histogram_kernel(
    const int32_t* __restrict__ topk_idx, int T, int k, int E,
    int32_t* __restrict__ tile_base, int32_t* __restrict__ slot_rank) {
  __shared__ unsigned long long bits[MOE_MAX_EXPERTS];
  const int tile = blockIdx.x;
  const int t0 = tile * kTileT;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) bits[e] = 0ull;
  __syncthreads();
  const int n = min(kTileT, T - t0) * k;
  const int32_t* ids = topk_idx + (size_t)t0 * k;
  for (int p = tid; p < n; p += 256) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicOr(&bits[e], 1ull << (p / k));
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256)
    tile_base[(size_t)tile * E + e] = __popcll(bits[e]);
  for (int p = tid; p < n; p += 256) {
    const int e = ids[p];
    const int tl = p / k;
    int r = -1;
    if (e >= 0 && e < E) r = __popcll(bits[e] & ((1ull << tl) - 1ull));
    slot_rank[(size_t)t0 * k + p] = r;
  }
}

// ------------------------------------------------------------------ scan

// Single workgroup of 1024 threads.  Thread (p, e) with p < parts owns a
// contiguous run of tiles of expert e.  Pass 1 sums the runs, the LDS scans
// give each run's start within its expert and the padded expert offsets,
// pass 2 overwrites every tile count with the first row of that
// (tile, expert) run: offsets[e] + tokens of e in earlier tiles.
__global__ __launch_bounds__(1024) void expert_scan_kernel(
    int32_t* __restrict__ tile_base, int ntiles, int E, int pad,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int part[1024];
  __shared__ int scan[1024];
  const int tid = threadIdx.x;
  int parts = 1024 / E;
  if (parts > ntiles) parts = ntiles;
  const int e = tid % E, p = tid / E;
  const bool active = p < parts;
  const int lo = active ? (int)((long long)p * ntiles / parts) : 0;
  const int hi = active ? (int)((long long)(p + 1) * ntiles / parts) : 0;

  int sum = 0;
  {
    int tl = lo;
    for (; tl + 8 <= hi; tl += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = tile_base[(size_t)(tl + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; tl < hi; ++tl) sum += tile_base[(size_t)tl * E + e];
  }
  if (active) part[p * E + e] = sum;
  __syncthreads();
  int padded = 0;
  if (tid < E) {
    int run = 0;
    for (int q = 0; q < parts; ++q) {
      const int v = part[q * E + tid];
      part[q * E + tid] = run;
      run += v;
    }
    counts[tid] = run;
    padded = (run + pad - 1) / pad * pad;
  }
  scan[tid] = padded;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  if (tid < E) offsets[tid + 1] = scan[tid];
  if (tid == 0) offsets[0] = 0;
  if (active) {
    int run = part[p * E + e] + (e == 0 ? 0 : scan[e - 1]);
    for (int tl = lo; tl < hi; ++tl) {
      const size_t i = (size_t)tl * E + e;
      const int c = tile_base[i];
      tile_base[i] = run;
      run += c;
    }
  }
}

// ------------------------------------------------------------------ launchers

template <typename XT>
static hipError_t launch_gate_typed(const XT* x, const XT* w, const float* bias,
                                    int T, int H, int E, int k, int32_t* idx,
                                    float* tw, float* dbg, hipStream_t s) {
  const int et = (E + 15) / 16;
  if (et <= 2) {
    const dim3 grid((T + 15) / 16);
    if (et == 1)
      hipLaunchKernelGGL((gate_topk_ksplit_kernel<XT, 1>), grid, dim3(256), 0,
                         s, x, w, bias, T, H, E, k, idx, tw, dbg);
    else
      hipLaunchKernelGGL((gate_topk_ksplit_kernel<XT, 2>), grid, dim3(256), 0,
                         s, x, w, bias, T, H, E, k, idx, tw, dbg);
    return hipGetLastError();
  }
  const dim3 grid((T + 63) / 64);
#define MOE_GATE_WIDE(ETV)                                                    \
  hipLaunchKernelGGL((gate_topk_wide_kernel<XT, ETV>), grid, dim3(256), 0, s, \
                     x, w, bias, T, H, E, k, idx, tw, dbg)
  if (et <= 4) MOE_GATE_WIDE(4);
  else if (et <= 8) MOE_GATE_WIDE(8);
  else if (et <= 16) MOE_GATE_WIDE(16);
  else if (et <= 24) MOE_GATE_WIDE(24);
  else MOE_GATE_WIDE(32);
#undef MOE_GATE_WIDE
  return hipGetLastError();
}

hipError_t launch_gate_topk(const void* x, const void* w, int xdt,
                            const float* bias, int T, int H, int E, int k,
                            int32_t* topk_idx, float* topk_w,
                            float* logits_dbg, hipStream_t s) {
  if (xdt == DT_BF16)
    return launch_gate_typed<uint16_t>((const uint16_t*)x, (const uint16_t*)w,
                                       bias, T, H, E, k, topk_idx, topk_w,
                                       logits_dbg, s);
  return launch_gate_typed<float>((const float*)x, (const float*)w, bias, T, H,
                                  E, k, topk_idx, topk_w, logits_dbg, s);
}

hipError_t launch_plan(const int32_t* topk_idx, int T, int k, int E, int pad,
                       int32_t* counts, int32_t* offsets, void* workspace,
                       hipStream_t s) {
  const int nt = num_tiles(T);
  int32_t* tile_base = (int32_t*)workspace;
  int32_t* slot_rank =
      (int32_t*)((unsigned char*)workspace + ws_tile_bytes(T, E));
  if (nt > 0) {
    hipLaunchKernelGGL(tile_histogram_kernel, dim3(nt), dim3(256), 0, s,
                       topk_idx, T, k, E, tile_base, slot_rank);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(expert_scan_kernel, dim3(1), dim3(1024), 0, s, tile_base,
                     nt, E, pad, counts, offsets);
  return hipGetLastError();
}

}  // namespace moe
