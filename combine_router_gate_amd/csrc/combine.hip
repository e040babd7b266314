// Weighted gather-combine back to token order, fused with the FarSkip
// dual residual update, for gfx950.
//
// Each token's output is the weighted sum of its selected experts' outputs
// with the router weights ("Efficient and Portable Mixture-of-Experts
// Communication", Introduction and Combine), and the accumulation is fused
// into the gather that collects them (same page, Sharding and Parallelism).
// The dual residual update follows the Instella-MoE article (where the dual
// residual streams are implemented): with MoE output = routed + shared,
//   residual_no_routed = residual + shared
//   residual           = residual + MoE output
// so the auxiliary stream never depends on the routed combine.
//
// Design for CDNA4: a token's row is split into groups of 128 16-byte
// chunks (64 with few tokens), one wavefront each, so the waves of a token
// run side by side.  Lanes 0..k-1 fetch the k (row, weight) pairs,
// broadcast to scalar registers; each lane then owns two groups of 8
// consecutive hidden elements (one with few tokens) and issues all their
// 16-byte row gathers plus the residual and shared loads before any
// arithmetic (20 independent loads in flight per lane at k = 8),
// accumulates in fp32 with j ascending (fmaf), adds shared then residual,
// rounds once to bf16 with the hardware converter and writes with streaming
// stores.  No floating-point atomics: every output element is produced by
// exactly one lane.  In-place use (residual_out == residual_in) is safe:
// each element is read before the same lane overwrites it.
#include "moe_device.h"
#include "moe_launch.h"

namespace moe {

// 8 consecutive elements of a row: one 16-byte vector of bf16 or two of fp32
template <int YT> struct Chunk8;
template <> struct Chunk8<1> { u32x4 a; };
template <> struct Chunk8<0> { u32x4 a, b; };

template <int YT>
__device__ __forceinline__ Chunk8<YT> load8(const unsigned char* __restrict__ row,
                                            int c) {
  Chunk8<YT> v;
  if constexpr (YT == 1) {
    v.a = ld16_stream(row + (size_t)c * 16);
  } else {
    v.a = ld16_stream(row + (size_t)c * 32);
    v.b = ld16_stream(row + (size_t)c * 32 + 16);
  }
  return v;
}
template <int YT>
__device__ __forceinline__ void unpack8(const Chunk8<YT>& v, float f[8]) {
  if constexpr (YT == 1) {
    unpack8_bf16(v.a, f);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = __uint_as_float(v.a[i]);
      f[4 + i] = __uint_as_float(v.b[i]);
    }
  }
}

// OUT: 0 = dual residual (bf16), 1 = routed-only bf16, 2 = routed-only fp32,
// 3 = main residual stream only (bf16; the auxiliary stream comes from
// farskip_aux_kernel).
// Each lane keeps U groups of 8 elements in flight: for k = 8 and U = 2 that
// is 2 * (8 gathers + shared + residual) 16-byte loads issued before any
// math.  U = 1 halves a wave's share of the row, so that few tokens can be
// spread over twice as many waves.  Workgroups of 8 waves (DeepSeek-V3
// prefill 503 -> 497 us against 4; 16 were slower).
template <int KMAX, int YT, int OUT, int U>
__global__ __launch_bounds__(512) void combine_kernel(
    const unsigned char* __restrict__ y, long long y_rows, int H,
    const int32_t* __restrict__ tok_row, const float* __restrict__ topk_w,
    int T, int k, const unsigned char* __restrict__ shared,
    const unsigned char* res_in, unsigned char* res_out,
    unsigned char* __restrict__ rnr, unsigned char* __restrict__ out,
    int hsplit) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // wave -> (token, part): hsplit waves share one token's hidden dimension
  // (interleaved groups of 64*U chunks)
  const int gw = blockIdx.x * (int)(blockDim.x >> 6) + wv;
  const int t = gw / hsplit, part = gw - t * hsplit;
  if (t >= T) return;

  int r = -1;
  float wt = 0.0f;
  if (lane < k) {
    const size_t s = (size_t)t * k + lane;
    r = tok_row[s];
    wt = topk_w != nullptr ? topk_w[s] : 1.0f;   // unit weights: plain sum
    if (r < 0 || (long long)r >= y_rows) r = -1;
  }
  int rj[KMAX];
  float wj[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    rj[j] = (j < k) ? __builtin_amdgcn_readlane(r, j) : -1;
    wj[j] = (j < k) ? __uint_as_float(__builtin_amdgcn_readlane(
                          __float_as_uint(wt), j))
                    : 0.0f;
  }
  const size_t yrowb = (size_t)H * (YT == 1 ? 2 : 4);
  const size_t trow = (size_t)t * H * 2;     // byte offset of token row, bf16
  const int nc8 = H / 8;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int c0 = part * 64 * U + lane; c0 < nc8; c0 += hsplit * 64 * U) {
    Chunk8<YT> g[U][KMAX];
    u32x4 shv[U], rsv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * 64;
      if (c < nc8) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (rj[j] >= 0) g[u][j] = load8<YT>(y + (size_t)rj[j] * yrowb, c);
        shv[u] = shared != nullptr ? ld16_stream(shared + trow + (size_t)c * 16) : z;
        if constexpr (OUT == 0 || OUT == 3)
          rsv[u] = ld16(res_in + trow + (size_t)c * 16);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * 64;
      if (c >= nc8) continue;
      float acc[8], sh[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (rj[j] >= 0) {
          float f[8];
          unpack8<YT>(g[u][j], f);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj[j], f[i], acc[i]);
        }
      }
      unpack8_bf16(shv[u], sh);
      if constexpr (OUT == 0 || OUT == 3) {
        float rs[8], o[8], a[8];
        unpack8_bf16(rsv[u], rs);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          o[i] = (acc[i] + sh[i]) + rs[i];
          a[i] = rs[i] + sh[i];
        }
        st16_stream(res_out + trow + (size_t)c * 16, pack8_bf16(o));
        if constexpr (OUT == 0)
          st16_stream(rnr + trow + (size_t)c * 16, pack8_bf16(a));
      } else {
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = acc[i] + sh[i];
        if constexpr (OUT == 1) {
          st16_stream(out + trow + (size_t)c * 16, pack8_bf16(o));
        } else {
          u32x4 v0, v1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v0[i] = __float_as_uint(o[i]);
            v1[i] = __float_as_uint(o[4 + i]);
          }
          unsigned char* p = out + (size_t)t * H * 4 + (size_t)c * 32;
          st16_stream(p, v0);
          st16_stream(p + 16, v1);
        }
      }
    }
  }
}

template <int KMAX, int YT, int U>
static void launch_combine_k(int om, dim3 grid, hipStream_t s,
                             const unsigned char* y, long long y_rows, int H,
                             const int32_t* tok_row, const float* w, int T,
                             int k, const unsigned char* sh,
                             const unsigned char* ri, unsigned char* ro,
                             unsigned char* rn, unsigned char* out, int hs) {
  if (om == 0)
    hipLaunchKernelGGL((combine_kernel<KMAX, YT, 0, U>), grid, dim3(512), 0, s,
                       y, y_rows, H, tok_row, w, T, k, sh, ri, ro, rn, out, hs);
  else if (om == 3)
    hipLaunchKernelGGL((combine_kernel<KMAX, YT, 3, U>), grid, dim3(512), 0, s,
                       y, y_rows, H, tok_row, w, T, k, sh, ri, ro, rn, out, hs);
  else if (om == 1)
    hipLaunchKernelGGL((combine_kernel<KMAX, YT, 1, U>), grid, dim3(512), 0, s,
                       y, y_rows, H, tok_row, w, T, k, sh, ri, ro, rn, out, hs);
  else
    hipLaunchKernelGGL((combine_kernel<KMAX, YT, 2, U>), grid, dim3(512), 0, s,
                       y, y_rows, H, tok_row, w, T, k, sh, ri, ro, rn, out, hs);
}


hipError_t launch_combine(const void* y, int ydt, int H, size_t y_rows,
                          const int32_t* tok_row, const float* topk_w, int T,
                          int k, const void* shared, const void* res_in,
                          void* res_out, void* rnr, void* out, int odt,
                          hipStream_t s) {
  // Every group of 64*U chunks of a token row is a wave of its own (the
  // waves of one token run side by side instead of one wave looping over
  // the row: DeepSeek-V3 prefill 535 -> 504 us, 7 waves per token); two
  // 64-lane chunks per lane step, or one when that leaves fewer than 2048
  // waves (few tokens)
  const int groups2 = (H / 8 + 127) / 128;
  const int u = (long long)T * groups2 >= 2048 ? 2 : 1;
  const int hs = u == 2 ? groups2 : (H / 8 + 63) / 64;
  const dim3 grid((unsigned)(((long long)T * hs + 7) / 8));
  const int om = res_in != nullptr ? (rnr != nullptr ? 0 : 3)
                                   : (odt == DT_BF16 ? 1 : 2);
  const unsigned char* yb = (const unsigned char*)y;
  const unsigned char* sh = (const unsigned char*)shared;
  const unsigned char* ri = (const unsigned char*)res_in;
  unsigned char* ro = (unsigned char*)res_out;
  unsigned char* rn = (unsigned char*)rnr;
  unsigned char* ob = (unsigned char*)out;
  const long long yr = (long long)y_rows;
#define MOE_COMB_U(KV, YV)                                                    \
  do {                                                                        \
    if (u == 2)                                                               \
      launch_combine_k<KV, YV, 2>(om, grid, s, yb, yr, H, tok_row, topk_w, T, \
                                  k, sh, ri, ro, rn, ob, hs);                 \
    else                                                                      \
      launch_combine_k<KV, YV, 1>(om, grid, s, yb, yr, H, tok_row, topk_w, T, \
                                  k, sh, ri, ro, rn, ob, hs);                 \
  } while (0)
#define MOE_COMB(KV)                                                          \
  do {                                                                        \
    if (ydt == DT_BF16) MOE_COMB_U(KV, 1);                                    \
    else MOE_COMB_U(KV, 0);                                                   \
  } while (0)
  if (k <= 1) MOE_COMB(1);
  else if (k <= 2) MOE_COMB(2);
  else if (k <= 4) MOE_COMB(4);
  else if (k <= 8) MOE_COMB(8);
  else MOE_COMB(16);
#undef MOE_COMB
#undef MOE_COMB_U
  return hipGetLastError();
}

// ------------------------------------------------------------------ FarSkip auxiliary stream

// residual_no_routed = bf16(residual + shared): the auxiliary stream of the
// dual residual update, which needs neither the router nor the routed
// combine and can therefore be produced before them (the next layer's
// attention reads this stream while the routed combine is still pending).
__global__ __launch_bounds__(256) void farskip_aux_kernel(
    const unsigned char* __restrict__ shared,
    const unsigned char* __restrict__ residual,
    unsigned char* __restrict__ rnr, long long n16) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (long long)gridDim.x * 256) {
    float sh[8], rs[8], a[8];
    const u32x4 z = {0u, 0u, 0u, 0u};
    unpack8_bf16(shared != nullptr ? ld16_stream(shared + i * 16) : z, sh);
    unpack8_bf16(ld16_stream(residual + i * 16), rs);
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = rs[q] + sh[q];
    st16_stream(rnr + i * 16, pack8_bf16(a));
  }
}

hipError_t launch_farskip_aux(const void* shared, const void* residual,
                              void* rnr, int T, int H, hipStream_t s) {
  // one 16-byte vector per thread (a grid-stride loop of 4096 workgroups
  // measured 125 us at DeepSeek-V3 prefill, this 111 us)
  const long long n16 = (long long)T * H / 8;
  long long blocks = (n16 + 255) / 256;
  if (blocks > 0x7fffffffLL) blocks = 0x7fffffffLL;
  hipLaunchKernelGGL(farskip_aux_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     s, (const unsigned char*)shared,
                     (const unsigned char*)residual, (unsigned char*)rnr, n16);
  return hipGetLastError();
}

// ------------------------------------------------------------------ backward

// Backward of the weighted combine routed[t] = sum_j w[t,j] * y[tok_row[t,j]]
// for an upstream gradient g = dL/d routed:
//   grad_y[tok_row[t,j]] = w[t,j] * g[t]            (bf16, one write per row)
//   grad_w[t,j]          = sum_h g[t,h] * y[tok_row[t,j],h]   (fp32)
// One wave per token; each lane keeps k partial dot products over its
// hidden elements, reduced across the wave in a fixed order at the end.
template <int KMAX, int YT>
__global__ __launch_bounds__(1024) void combine_backward_kernel(
    const unsigned char* __restrict__ g, const unsigned char* __restrict__ y,
    long long y_rows, int H, const int32_t* __restrict__ tok_row,
    const float* __restrict__ topk_w, int T, int k,
    unsigned char* __restrict__ grad_y, float* __restrict__ grad_w, int hs) {
  // hs waves of one workgroup share a token's hidden dimension (interleaved
  // groups of 64 chunks); their partial dot products meet in LDS and are
  // summed in wave order, so grad_w does not depend on timing.
  __shared__ float part[16][KMAX];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int tpb = (int)(blockDim.x >> 6) / hs;
  const int t = blockIdx.x * tpb + wv / hs, p = wv % hs;
  const bool live = t < T;
  int r = -1;
  float wt = 0.0f;
  if (live && lane < k) {
    const size_t s = (size_t)t * k + lane;
    r = tok_row[s];
    wt = topk_w[s];
    if (r < 0 || (long long)r >= y_rows) r = -1;
  }
  int rj[KMAX];
  float wj[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    rj[j] = (j < k) ? __builtin_amdgcn_readlane(r, j) : -1;
    wj[j] = (j < k) ? __uint_as_float(__builtin_amdgcn_readlane(
                          __float_as_uint(wt), j))
                    : 0.0f;
  }
  const size_t yrowb = (size_t)H * (YT == 1 ? 2 : 4);
  const size_t trow = (size_t)(live ? t : 0) * H * 2;
  const int nc8 = live ? H / 8 : 0;
  float dot[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) dot[j] = 0.0f;
  for (int c = p * 64 + lane; c < nc8; c += hs * 64) {
    // the gradient chunk and all k row chunks are loaded before any of them
    // is used, so they are in flight together
    const u32x4 gv = ld16_stream(g + trow + (size_t)c * 16);
    Chunk8<YT> yv[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (rj[j] >= 0) {
        const unsigned char* yr = y + (size_t)rj[j] * yrowb;
        if constexpr (YT == 1) {
          yv[j].a = ld16(yr + (size_t)c * 16);
        } else {
          yv[j].a = ld16(yr + (size_t)c * 32);
          yv[j].b = ld16(yr + (size_t)c * 32 + 16);
        }
      }
    float gf[8];
    unpack8_bf16(gv, gf);
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (rj[j] < 0) continue;
      float yf[8], d[8];
      unpack8<YT>(yv[j], yf);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dot[j] = fmaf(gf[i], yf[i], dot[j]);
        d[i] = wj[j] * gf[i];
      }
      st16_stream(grad_y + (size_t)rj[j] * H * 2 + (size_t)c * 16,
                  pack8_bf16(d));
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    float v = dot[j];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    if (lane == 0) part[wv][j] = v;
  }
  __syncthreads();
  if (live && p == 0 && lane < k) {
    float v = 0.0f;
    for (int q = 0; q < hs; ++q) v += part[wv + q][lane];
    grad_w[(size_t)t * k + lane] = v;
  }
}

hipError_t launch_combine_backward(const void* g, const void* y, int ydt,
                                   int H, size_t y_rows,
                                   const int32_t* tok_row,
                                   const float* topk_w, int T, int k,
                                   void* grad_y, float* grad_w,
                                   hipStream_t s) {
  // waves per token: a power of two up to 16, for up to ~16384 waves
  // (MoonEP 8192 tokens of 768: 42 -> 39.5 us)
  const int groups = (H / 8 + 63) / 64;
  int hs = 1;
  while (hs < 16 && 2 * hs <= groups && (long long)T * hs < 16384) hs *= 2;
  const int waves = hs > 4 ? hs : 4;
  const int tpb = waves / hs;
  const dim3 grid((unsigned)((T + tpb - 1) / tpb)), block(64 * waves);
  const unsigned char* gb = (const unsigned char*)g;
  const unsigned char* yb = (const unsigned char*)y;
  unsigned char* dyb = (unsigned char*)grad_y;
  const long long yr = (long long)y_rows;
#define MOE_CBWD(KV)                                                           \
  do {                                                                         \
    if (ydt == DT_BF16)                                                        \
      hipLaunchKernelGGL((combine_backward_kernel<KV, 1>), grid, block, 0, s,  \
                         gb, yb, yr, H, tok_row, topk_w, T, k, dyb, grad_w,    \
                         hs);                                                  \
    else                                                                       \
      hipLaunchKernelGGL((combine_backward_kernel<KV, 0>), grid, block, 0, s,  \
                         gb, yb, yr, H, tok_row, topk_w, T, k, dyb, grad_w,    \
                         hs);                                                  \
  } while (0)
  if (k <= 1) MOE_CBWD(1);
  else if (k <= 2) MOE_CBWD(2);
  else if (k <= 4) MOE_CBWD(4);
  else if (k <= 8) MOE_CBWD(8);
  else MOE_CBWD(16);
#undef MOE_CBWD
  return hipGetLastError();
}

}  // namespace moe
