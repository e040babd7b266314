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
// Design for CDNA4: one wavefront per token.  Lanes 0..k-1 fetch the k
// (row, weight) pairs, broadcast to scalar registers; each lane then owns
// two groups of 8 consecutive hidden elements per step and issues all their
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

// OUT: 0 = dual residual (bf16), 1 = routed-only bf16, 2 = routed-only fp32.
// Each lane keeps U = 2 groups of 8 elements in flight: for k = 8 that is
// 2 * (8 gathers + shared + residual) 16-byte loads issued before any math.
template <int KMAX, int YT, int OUT>
__global__ __launch_bounds__(256) void combine_kernel(
    const unsigned char* __restrict__ y, long long y_rows, int H,
    const int32_t* __restrict__ tok_row, const float* __restrict__ topk_w,
    int T, int k, const unsigned char* __restrict__ shared,
    const unsigned char* res_in, unsigned char* res_out,
    unsigned char* __restrict__ rnr, unsigned char* __restrict__ out) {
  constexpr int U = 2;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;

  int r = -1;
  float wt = 0.0f;
  if (lane < k) {
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
  const size_t trow = (size_t)t * H * 2;     // byte offset of token row, bf16
  const int nc8 = H / 8;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int c0 = lane; c0 < nc8; c0 += 64 * U) {
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
        if constexpr (OUT == 0) rsv[u] = ld16(res_in + trow + (size_t)c * 16);
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
      if constexpr (OUT == 0) {
        float rs[8], o[8], a[8];
        unpack8_bf16(rsv[u], rs);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          o[i] = (acc[i] + sh[i]) + rs[i];
          a[i] = rs[i] + sh[i];
        }
        st16_stream(res_out + trow + (size_t)c * 16, pack8_bf16(o));
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

template <int KMAX, int YT>
static void launch_combine_k(int om, dim3 grid, hipStream_t s,
                             const unsigned char* y, long long y_rows, int H,
                             const int32_t* tok_row, const float* w, int T,
                             int k, const unsigned char* sh,
                             const unsigned char* ri, unsigned char* ro,
                             unsigned char* rn, unsigned char* out) {
  if (om == 0)
    hipLaunchKernelGGL((combine_kernel<KMAX, YT, 0>), grid, dim3(256), 0, s, y,
                       y_rows, H, tok_row, w, T, k, sh, ri, ro, rn, out);
  else if (om == 1)
    hipLaunchKernelGGL((combine_kernel<KMAX, YT, 1>), grid, dim3(256), 0, s, y,
                       y_rows, H, tok_row, w, T, k, sh, ri, ro, rn, out);
  else
    hipLaunchKernelGGL((combine_kernel<KMAX, YT, 2>), grid, dim3(256), 0, s, y,
                       y_rows, H, tok_row, w, T, k, sh, ri, ro, rn, out);
}

hipError_t launch_combine(const void* y, int ydt, int H, size_t y_rows,
                          const int32_t* tok_row, const float* topk_w, int T,
                          int k, const void* shared, const void* res_in,
                          void* res_out, void* rnr, void* out, int odt,
                          hipStream_t s) {
  const dim3 grid((T + 3) / 4);
  const int om = res_in != nullptr ? 0 : (odt == DT_BF16 ? 1 : 2);
  const unsigned char* yb = (const unsigned char*)y;
  const unsigned char* sh = (const unsigned char*)shared;
  const unsigned char* ri = (const unsigned char*)res_in;
  unsigned char* ro = (unsigned char*)res_out;
  unsigned char* rn = (unsigned char*)rnr;
  unsigned char* ob = (unsigned char*)out;
  const long long yr = (long long)y_rows;
#define MOE_COMB(KV)                                                          \
  do {                                                                        \
    if (ydt == DT_BF16)                                                       \
      launch_combine_k<KV, 1>(om, grid, s, yb, yr, H, tok_row, topk_w, T, k,  \
                              sh, ri, ro, rn, ob);                            \
    else                                                                      \
      launch_combine_k<KV, 0>(om, grid, s, yb, yr, H, tok_row, topk_w, T, k,  \
                              sh, ri, ro, rn, ob);                            \
  } while (0)
  if (k <= 1) MOE_COMB(1);
  else if (k <= 2) MOE_COMB(2);
  else if (k <= 4) MOE_COMB(4);
  else if (k <= 8) MOE_COMB(8);
  else MOE_COMB(16);
#undef MOE_COMB
  return hipGetLastError();
}

}  // namespace moe
