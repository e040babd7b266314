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
//    Softmax and top-k run on-chip, so the logits never touch HBM (only fp32
//    partial sums of a split hidden dimension do).
//  * E >= 64, bf16: the hidden dimension is split into S ranges so that
//    about 256 workgroups run; gate_partial_lds_kernel (4096 tokens and
//    more: 128 tokens x all experts per workgroup, both operands staged
//    through LDS) or gate_partial_kernel (up to 512 tokens with one group
//    of 64 experts per workgroup) writes the partial logits, and
//    gate_reduce_quad_kernel (gate_reduce_small_kernel up to 512 tokens)
//    sums them in range order and selects the top-k.  Where a split
//    would not pay, gate_topk_v2_kernel does all of it in one pass.  A
//    narrow gate (weight under 1 MiB, 4096 to 32768 tokens) skips the
//    split: gate_topk_narrow_kernel runs 32 tokens x all experts per
//    workgroup, each streaming the whole weight from L2 through LDS, with
//    the top-k in its epilogue.  Above 512 experts (bf16) the partial
//    logits come in expert groups of 256 and the top-k of a token takes a
//    whole wave.  x is read with ordinary (allocating) loads, so the
//    dispatch that reads it next finds much of it still in the
//    memory-attached cache.
//  * E < 64 (memory-bound gate): the 4 waves split the hidden dimension of a
//    16-token tile and reduce their partial logits through LDS in a fixed
//    order, so four times as many workgroups stream x.
//  * Top-k: the 16 lanes of a lane group hold all logits of one token; k
//    rounds of a 16-lane max over 64-bit keys (order-preserving logit key,
//    then inverted expert id) give the lowest-index tie-break exactly; for
//    4 <= k <= 8 each lane first sorts its 8 largest keys, so a round only
//    compares list heads.
//    Weights are exp(l_j - l_max) / sum over the chosen, i.e. the full
//    softmax renormalised over the chosen experts (the all-expert
//    denominator cancels).
//  * Histogram: per 64-token tile, an LDS bitmap per expert (bit = token)
//    assembled with ds_or_b64; its popcount is the tile count and the
//    popcount of the bits below a token is that token's rank, which fixes a
//    stable, deterministic slot order with no global atomics.
//  * Scan: the [tiles, E] counts become, in place, the first row of every
//    (tile, expert) run.  After a split or narrow gate one workgroup per
//    group of 16 tiles does it from per-group expert totals that the
//    histogram producers accumulate; otherwise one workgroup scans all
//    tiles; up to 512 tokens one workgroup plans everything in LDS.
#include "scatter_device.h"

#include <algorithm>
#include <atomic>

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

// Slot of 16-byte piece p of row r in a row-major LDS tile of 128-byte rows
// is p ^ gate_lds_swz(r): the coalesced writes (8 lanes per row) and the
// fragment reads (16 rows, one piece) then touch distinct banks on gfx950,
// whose ds_*_b128 grouping a plain p ^ (r & 7) leaves 2-way conflicted.
__device__ __forceinline__ int gate_lds_swz(int r) {
  return (r & 7) ^ ((r >> 3) & 1);
}

// The histogram producers after a split gate accumulate per-group expert
// totals with integer atomics; the gate kernel, which runs first in the same
// call, clears them (n ints, spread over every thread of the grid).
__device__ __forceinline__ void clear_group_totals(int32_t* __restrict__ g,
                                                   int n) {
  if (g == nullptr) return;
  const long long bid = blockIdx.x + (long long)gridDim.x *
                                         (blockIdx.y + (long long)gridDim.y *
                                                           blockIdx.z);
  const long long nthr =
      (long long)gridDim.x * gridDim.y * gridDim.z * blockDim.x;
  for (long long i = bid * blockDim.x + threadIdx.x; i < n; i += nthr)
    g[i] = 0;
}

// ------------------------------------------------------------------ top-k

// Top-k of one token per 16-lane group.  Lane c of the group holds the
// logits of experts 16*et + c in v[et] (bias already added).  Each logit
// becomes a 64-bit key (order-preserving logit key, then inverted expert
// id), built once; padded experts get key 0.  k rounds of a 16-lane max
// pick the largest logit, lowest index first on ties.  For 4 <= k <= 8
// (and 8+ keys per lane) each lane first sorts its 8 largest keys (no lane
// can supply more than k choices) and a round's winner lane drops its head;
// otherwise (and where SORT8 is off: the sorted list does not fit the
// registers of 1024-thread workgroups beyond 16 keys per lane) the winner is
// removed by clearing its high word, which leaves it below every
// real key (the key of any non-NaN logit has a non-zero high word).  Lane j
// of the group writes the j-th choice and its renormalised weight.
// Lane c of a 16-lane group holds expert 16 et + c in v[et], or with QUAD
// expert 64 (et / 4) + 4 c + et % 4 (four consecutive experts per 16-byte
// load).
template <bool QUAD>
__device__ __forceinline__ int topk_expert(int et, int c) {
  return QUAD ? 64 * (et >> 2) + 4 * c + (et & 3) : et * 16 + c;
}

// Compare-exchange of 64-bit keys: the larger to a, the smaller to b.
__device__ __forceinline__ void ce_desc(unsigned long long& a,
                                        unsigned long long& b) {
  const bool sw = b > a;
  const unsigned long long hi = sw ? b : a, lo = sw ? a : b;
  a = hi;
  b = lo;
}
// Keys o .. o + 7 in descending order (Batcher's odd-even merge sort, 19
// compare-exchanges).
template <int N>
__device__ __forceinline__ void sort8_desc(unsigned long long (&q)[N], int o) {
  ce_desc(q[o + 0], q[o + 1]); ce_desc(q[o + 2], q[o + 3]);
  ce_desc(q[o + 4], q[o + 5]); ce_desc(q[o + 6], q[o + 7]);
  ce_desc(q[o + 0], q[o + 2]); ce_desc(q[o + 1], q[o + 3]);
  ce_desc(q[o + 4], q[o + 6]); ce_desc(q[o + 5], q[o + 7]);
  ce_desc(q[o + 1], q[o + 2]); ce_desc(q[o + 5], q[o + 6]);
  ce_desc(q[o + 0], q[o + 4]); ce_desc(q[o + 1], q[o + 5]);
  ce_desc(q[o + 2], q[o + 6]); ce_desc(q[o + 3], q[o + 7]);
  ce_desc(q[o + 2], q[o + 4]); ce_desc(q[o + 3], q[o + 5]);
  ce_desc(q[o + 1], q[o + 2]); ce_desc(q[o + 3], q[o + 4]);
  ce_desc(q[o + 5], q[o + 6]);
}
// This lane's 8 largest keys in descending order (zeros past its ET keys):
// groups of 8 (the last padded with zeros) sorted, then merged pairwise
// keeping the top 8 (the largest 8 of two descending lists are
// max(a_i, b_{7-i}), a bitonic sequence that 12 compare-exchanges sort).
template <int ET>
__device__ __forceinline__ void lane_top8(const unsigned long long (&key)[ET],
                                          unsigned long long (&L)[8]) {
  constexpr int NG = (ET + 7) / 8;
  unsigned long long q[8 * NG];
#pragma unroll
  for (int i = 0; i < 8 * NG; ++i) q[i] = i < ET ? key[i] : 0ull;
#pragma unroll
  for (int g = 0; g < NG; ++g) sort8_desc(q, 8 * g);
#pragma unroll
  for (int i = 0; i < 8; ++i) L[i] = q[i];
#pragma unroll
  for (int g = 1; g < NG; ++g) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned long long b = q[8 * g + 7 - i];
      L[i] = b > L[i] ? b : L[i];
    }
    ce_desc(L[0], L[4]); ce_desc(L[1], L[5]);
    ce_desc(L[2], L[6]); ce_desc(L[3], L[7]);
    ce_desc(L[0], L[2]); ce_desc(L[1], L[3]);
    ce_desc(L[4], L[6]); ce_desc(L[5], L[7]);
    ce_desc(L[0], L[1]); ce_desc(L[2], L[3]);
    ce_desc(L[4], L[5]); ce_desc(L[6], L[7]);
  }
}

template <int ET, bool QUAD = false, bool SORT8 = true>
__device__ __forceinline__ void topk_select_write(
    const float (&v)[ET], int t, int T, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    unsigned long long* tile_bits = nullptr, int* tile_sel = nullptr,
    int tl = 0) {
  const int c = threadIdx.x & 15;
  unsigned long long key[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et) {
    const int e = topk_expert<QUAD>(et, c);
    const uint32_t hi = e < E ? f32_order_key(v[et]) : 0u;
    key[et] = ((unsigned long long)hi << 32) | (0xffffffffu - (uint32_t)e);
  }
  int sel_e[MOE_MAX_TOPK];
  float sel_v[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    sel_e[j] = 0;
    sel_v[j] = 0.0f;
  }
  // with 8 or more keys per lane and 4 <= k <= 8 (where the one-time sort
  // costs fewer instructions than k full passes over the keys): a lane can
  // supply at most k of the choices, so its 8 largest keys are sorted once
  // and each round's winner lane drops its head
  if (SORT8 && ET >= 8 && k >= 4 && k <= 8) {
    unsigned long long L[8];
    lane_top8<ET>(key, L);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        const unsigned long long best = max16_u64(L[0]);
        const uint32_t blo = (uint32_t)best;
        const bool win = (uint32_t)L[0] == blo;
#pragma unroll
        for (int i = 0; i < 7; ++i) L[i] = win ? L[i + 1] : L[i];
        L[7] = win ? 0ull : L[7];
        sel_e[j] = (int)(0xffffffffu - blo);
        sel_v[j] = f32_from_order_key((uint32_t)(best >> 32));
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k) {
        unsigned long long best = key[0];
#pragma unroll
        for (int et = 1; et < ET; ++et) best = key[et] > best ? key[et] : best;
        best = max16_u64(best);
        const uint32_t blo = (uint32_t)best;
#pragma unroll
        for (int et = 0; et < ET; ++et)
          if ((uint32_t)key[et] == blo) key[et] &= 0xffffffffull;
        sel_e[j] = (int)(0xffffffffu - blo);
        sel_v[j] = f32_from_order_key((uint32_t)(best >> 32));
      }
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
        if (tile_bits != nullptr) {
          atomicOr(&tile_bits[sel_e[j]], 1ull << tl);
          tile_sel[tl * MOE_MAX_TOPK + j] = sel_e[j];
        }
      }
    }
  }
}

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
    topk_select_write<ET>(v, t, T, E, k, topk_idx, topk_w);
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
      frag_load<XT>(anext[s], xrow + kk, arow_ok && kk < H, false);
    }
  };

  load_w(0);
  load_a(0);
  for (int ch = 0; ch < nchunks; ++ch) {
    lds_barrier();
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int p = tid + 256 * i;
      st16(wlds + (p >> 3) * ROWB + (p & 7) * 16, wreg[i]);
    }
    lds_barrier();
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

// ------------------------------------------------------------------ gate v2, bf16, E >= 64

// One workgroup = 4 waves = 64 tokens.  Wave w owns all 64 tokens and the
// EPW expert tiles [w*EPW, (w+1)*EPW) (16 experts each), i.e. a 64 x 16*EPW
// block of logits in 4*EPW MFMA accumulators, so each x fragment read from
// LDS feeds EPW MFMAs and each gate-weight fragment feeds 4.
//
// The hidden dimension advances in super-steps of 128: lane group g =
// lane/16 owns k in [K0 + 32g, K0 + 32g + 32) as four 8-element pieces, one
// per 16x16x32 MFMA; x and W use the same (g, piece) -> k map, so each lane
// reads 64 contiguous bytes of every row it touches.
//  * x: the workgroup loads the [64 tokens x 128 k] tile (16 KB, 64 B per
//    thread) D super-steps ahead into a register ring and stores it into one
//    of two LDS slots right before use.  Within a slot, 16-byte piece p of
//    row r sits at position p ^ gate_lds_swz(r), so the 16 rows read by an
//    MFMA operand fall into distinct banks.
//  * W: each wave loads its own B fragments from global memory (the gate
//    weight stays L2-resident while x streams past it) into a D-deep
//    register ring.
// Every load in the pipeline is unconditional and unmasked (addresses
// clamped into the arrays), so the compiler counts outstanding loads exactly
// instead of draining them; out-of-range x (a token past T or k >= H) is
// zeroed only when the tile is written to LDS, after the load has landed.
// Out-of-range W then multiplies zeros (k >= H) or belongs to a padded
// expert that the top-k ignores.  One LDS-only barrier per super-step.
// Afterwards the logits go through LDS so each 16-lane group sees all
// experts of one token for the top-k, and the tile's expert bitmaps give
// its histogram and slot ranks.
template <int EPW, int PQ, int D>
__global__ __launch_bounds__(256, 1) void gate_topk_v2_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const float* __restrict__ bias, int T, int H, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits_dbg, int32_t* __restrict__ tile_base,
    int32_t* __restrict__ slot_rank) {
  constexpr int ET = 4 * EPW;              // expert tiles of the workgroup
  constexpr int EP = 16 * ET;              // padded experts
  constexpr int LROW = EP + 4;             // logits row stride (floats)
  constexpr int KS = 32 * PQ;              // k per super-step
  constexpr int RB = 2 * KS;               // bytes of one x row per step
  constexpr int NP = 4 * PQ;               // 16-byte pieces per row
  static_assert(NP == 8, "the LDS swizzle assumes 128-byte rows");
  constexpr int XSLOT = 64 * RB;           // bytes of one x slot
  constexpr int LDS_BYTES = (64 * LROW * 4 > 2 * XSLOT) ? 64 * LROW * 4 : 2 * XSLOT;
  __shared__ __align__(16) unsigned char lds[LDS_BYTES];
  __shared__ unsigned long long tile_bits[EP];     // token bitmap per expert
  __shared__ int tile_sel[64 * MOE_MAX_TOPK];      // chosen experts

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int t0 = blockIdx.x * 64;
  const int nss = (H + KS - 1) / KS;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int e = tid; e < EP; e += 256) tile_bits[e] = 0ull;

  // x tile loader: thread covers row tid/4, pieces PQ*(tid%4) .. +PQ-1
  const int xr = tid >> 2, xp = (tid & 3) * PQ;
  const bool xrow_ok = t0 + xr < T;
  const uint16_t* xrow = x + (size_t)(xrow_ok ? t0 + xr : T - 1) * H;
  const uint16_t* wrow[EPW];
#pragma unroll
  for (int et = 0; et < EPW; ++et) {
    const int e = (wv * EPW + et) * 16 + c16;
    wrow[et] = w + (size_t)(e < E ? e : E - 1) * H;
  }

  u32x4 xreg[D][PQ];
  u32x4 wreg[D][EPW][PQ];
  auto load_x = [&](int i, u32x4 (&dst)[PQ]) {
#pragma unroll
    for (int q = 0; q < PQ; ++q) {
      const int kk = i * KS + (xp + q) * 8;
      dst[q] = ld16(xrow + (kk < H ? kk : H - 8));
    }
  };
  auto load_w = [&](int i, u32x4 (&dst)[EPW][PQ]) {
#pragma unroll
    for (int et = 0; et < EPW; ++et)
#pragma unroll
      for (int q = 0; q < PQ; ++q) {
        const int kk = i * KS + g * (8 * PQ) + q * 8;
        dst[et][q] = ld16(wrow[et] + (kk < H ? kk : H - 8));
      }
  };

  f32x4 acc[4][EPW];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int et = 0; et < EPW; ++et) acc[tt][et] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int j = 0; j < D; ++j) {
    load_x(j, xreg[j]);
    load_w(j, wreg[j]);
  }

  // steps past the end (up to D-1 when nss % D != 0) multiply zeros
  for (int i0 = 0; i0 < nss; i0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int i = i0 + j;
      unsigned char* slot = lds + (i & 1) * XSLOT;
#pragma unroll
      for (int q = 0; q < PQ; ++q) {
        const bool ok = xrow_ok && i * KS + (xp + q) * 8 < H;
        st16(slot + xr * RB + (((xp + q) ^ gate_lds_swz(xr)) * 16),
             ok ? xreg[j][q] : z);
      }
      lds_barrier();
      load_x(i + D, xreg[j]);
#pragma unroll
      for (int q = 0; q < PQ; ++q) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int r = tt * 16 + c16;
          const int p = g * PQ + q;
          Frag<uint16_t> a;
          a.v = *reinterpret_cast<const u32x4*>(slot + r * RB + ((p ^ gate_lds_swz(r)) * 16));
#pragma unroll
          for (int et = 0; et < EPW; ++et) {
            Frag<uint16_t> b;
            b.v = wreg[j][et][q];
            acc[tt][et] = mfma_step(a, b, acc[tt][et]);
          }
        }
      }
      load_w(i + D, wreg[j]);
    }
  }

  // logits -> LDS [64 tokens][LROW] (bias added), then top-k per token
  __syncthreads();
  float* lg = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int et = 0; et < EPW; ++et) {
      const int e = (wv * EPW + et) * 16 + c16;
      const float b = (bias != nullptr && e < E) ? bias[e] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) lg[(tt * 16 + g * 4 + i) * LROW + e] = acc[tt][et][i] + b;
    }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int tl = wv * 16 + pass * 4 + g;
    const int t = t0 + tl;
    float v[ET];
#pragma unroll
    for (int et = 0; et < ET; ++et) {
      const int e = et * 16 + c16;
      v[et] = lg[tl * LROW + e];
      if (logits_dbg != nullptr && t < T && e < E)
        logits_dbg[(size_t)t * E + e] = v[et];
    }
    topk_select_write<ET>(v, t, T, E, k, topk_idx, topk_w, tile_bits,
                          tile_sel, tl);
  }
  // the tile's histogram and slot ranks (as tile_histogram_kernel does)
  __syncthreads();
  for (int e = tid; e < E; e += 256)
    tile_base[(size_t)blockIdx.x * E + e] = __popcll(tile_bits[e]);
  const int n = min(64, T - t0) * k;
  for (int q = tid; q < n; q += 256) {
    const int tl = q / k, j = q - tl * k;
    const int e = tile_sel[tl * MOE_MAX_TOPK + j];
    slot_rank[(size_t)t0 * k + q] = __popcll(tile_bits[e] & ((1ull << tl) - 1ull));
  }
}

// One pass of gate and top-k for a narrow gate (E * H small enough that
// every workgroup can stream the whole gate weight from L2): 32 tokens x
// all experts per workgroup of 8 waves, so there are twice as many
// workgroups as 64-token tiles and no partial logits go through HBM.  Per
// 64-wide k step both operands reach LDS through direct global->LDS copies
// (8 lanes per 128-byte row segment, 8 rows per copy; a lane fetches source
// piece (l & 7) ^ gate_lds_swz(row), so the row swizzle of the other gate
// kernels holds) into two stages: step i + 1 is copied while step i is
// computed, then one wait plus barrier hands the stages over (per wave 2 EPW
// weight groups, plus one x group on waves 0..3).  Wave wv owns expert
// tiles EPW wv .. +EPW (16 experts each) for both 16-token halves.  The
// logits then go through LDS so each 16-lane group holds one token's
// experts for the top-k (one token per group, one pass).  The kernel clears
// the per-group totals that the tile histogram of the same call
// accumulates.  Requires H % 64 == 0 and byte offsets of x and w below 2^32.
template <int EPW>
__global__ __launch_bounds__(512, 1) void gate_topk_narrow_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const float* __restrict__ bias, int T, int H, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits_dbg, int32_t* __restrict__ gzero,
    int gzero_n) {
  clear_group_totals(gzero, gzero_n);
  constexpr int TOK = 32;
  constexpr int ET = 8 * EPW;              // expert tiles of the workgroup
  constexpr int EP = 16 * ET;              // padded experts
  constexpr int LROW = EP + 4;             // logits row stride (floats)
  constexpr int XS = TOK * 128;            // bytes of x in one stage
  constexpr int STG = XS + EP * 128;       // bytes of one stage
  constexpr int WPW = 2 * EPW;             // weight copies per wave and step
  constexpr int LDS_BYTES = (TOK * LROW * 4 > 2 * STG) ? TOK * LROW * 4 : 2 * STG;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int t0 = blockIdx.x * TOK;
  const int nss = H / 64;
  const int lr = lane >> 3;
  const bool xwave = wv < 4;               // copies x rows 8 wv .. +7

  // byte offsets of this lane's source pieces (step 0); lane l copies piece
  // slot l & 7 of row l >> 3 of its 8-row group
  uint32_t xoff, woff[WPW];
  {
    const int r = 8 * (wv & 3) + lr;
    const uint32_t row = (uint32_t)min(t0 + r, T - 1);
    xoff = row * (uint32_t)H * 2u + (uint32_t)(((lane & 7) ^ gate_lds_swz(r)) * 16);
  }
#pragma unroll
  for (int m = 0; m < WPW; ++m) {
    const int r = 8 * (wv + 8 * m) + lr;
    const uint32_t row = (uint32_t)min(r, E - 1);
    woff[m] = row * (uint32_t)H * 2u + (uint32_t)(((lane & 7) ^ gate_lds_swz(r)) * 16);
  }
  auto copy_step = [&](int i, unsigned char* stage) {
    const unsigned char* xb = reinterpret_cast<const unsigned char*>(x) + (size_t)i * 128;
    const unsigned char* wb = reinterpret_cast<const unsigned char*>(w) + (size_t)i * 128;
    if (xwave) copy_to_lds16(xb, xoff, lds_addr(stage + wv * 1024));
#pragma unroll
    for (int m = 0; m < WPW; ++m)
      copy_to_lds16(wb, woff[m], lds_addr(stage + XS + (wv + 8 * m) * 1024));
  };

  f32x4 acc[2][EPW];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int et = 0; et < EPW; ++et) acc[tt][et] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragments: row r of the stage, piece 2 g + q
  auto frag = [&](const unsigned char* stage, int r, int q) {
    Frag<uint16_t> f;
    f.v = *reinterpret_cast<const u32x4*>(stage + r * 128 + (((2 * g + q) ^ gate_lds_swz(r)) * 16));
    return f;
  };
  auto compute = [&](const unsigned char* stage) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      Frag<uint16_t> a[2], b[EPW];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) a[tt] = frag(stage, tt * 16 + c16, q);
#pragma unroll
      for (int et = 0; et < EPW; ++et)
        b[et] = frag(stage, TOK + (wv * EPW + et) * 16 + c16, q);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int et = 0; et < EPW; ++et) acc[tt][et] = mfma_step(a[tt], b[et], acc[tt][et]);
    }
  };

  copy_step(0, lds);
  copies_barrier();
  for (int i = 0; i < nss; ++i) {
    if (i + 1 < nss) copy_step(i + 1, lds + ((i + 1) & 1) * STG);
    compute(lds + (i & 1) * STG);
    copies_barrier();
  }

  // logits -> LDS [32 tokens][LROW] (bias added), then top-k per token
  float* lg = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int et = 0; et < EPW; ++et) {
      const int e = (wv * EPW + et) * 16 + c16;
      const float b = (bias != nullptr && e < E) ? bias[e] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) lg[(tt * 16 + g * 4 + i) * LROW + e] = acc[tt][et][i] + b;
    }
  __syncthreads();
  const int tl = wv * 4 + g;
  const int t = t0 + tl;
  float v[ET];
#pragma unroll
  for (int et = 0; et < ET; ++et) {
    const int e = et * 16 + c16;
    v[et] = lg[tl * LROW + e];
    if (logits_dbg != nullptr && t < T && e < E)
      logits_dbg[(size_t)t * E + e] = v[et];
  }
  topk_select_write<ET>(v, t, T, E, k, topk_idx, topk_w);
}

// ------------------------------------------------------------------ gate, split over H

// Partial logits over one range of the hidden dimension, for shapes where
// one workgroup per 64-token tile cannot fill the chip (few tokens): the
// grid is (token tiles of 16*TT, hidden ranges of KR, expert groups of
// 64*EPW), each workgroup runs the same pipeline as gate_topk_v2_kernel
// over [k_lo, k_lo + KR) and writes its fp32 partial logits
// partial[ks][t][e] (row stride eps >= 64*EPW*gridDim.z).
// gate_reduce_quad_kernel / gate_reduce_small_kernel add the ranges in
// ascending order.  Expert groups let few tokens spread over many
// workgroups with fewer hidden ranges (fewer partial logits to add).
// Workgroup (bx, by, bz) of that grid (256 threads).
template <int EPW, int TT, int PQ, int D, int DX = D>
__device__ __forceinline__ void gate_partial_block(
    int bx, int by, int bz, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ w, int T, int H, int E, int KR, int eps,
    float* __restrict__ partial) {
  const int e0 = bz * 64 * EPW;            // first expert of the group
  constexpr int TTOK = 16 * TT;            // tokens of the workgroup
  constexpr int KS = 32 * PQ;              // k per super-step
  constexpr int RB = 2 * KS;               // bytes of one x row per step
  constexpr int NP = 4 * PQ;               // 16-byte pieces per row
  static_assert(NP == 8, "the LDS swizzle assumes 128-byte rows");
  constexpr int XSLOT = TTOK * RB;         // bytes of one x slot
  constexpr int XPT = TTOK * NP / 256;     // x pieces per thread per step
  static_assert(XPT >= 1 && TTOK * NP % 256 == 0, "tile too small");
  __shared__ __align__(16) unsigned char lds[2 * XSLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int t0 = bx * TTOK;
  const int ks = by;
  const int k_lo = ks * KR;
  const int k_hi = min(H, k_lo + KR);
  const int nss = (k_hi - k_lo + KS - 1) / KS;
  const u32x4 z = {0u, 0u, 0u, 0u};

  int xr[XPT], xp[XPT];
  bool xrow_ok[XPT];
  const uint16_t* xsrc[XPT];
#pragma unroll
  for (int m = 0; m < XPT; ++m) {
    const int u = tid + 256 * m;
    xr[m] = u / NP;
    xp[m] = u % NP;
    xrow_ok[m] = t0 + xr[m] < T;
    xsrc[m] = x + (size_t)(xrow_ok[m] ? t0 + xr[m] : T - 1) * H;
  }
  const uint16_t* wrow[EPW];
#pragma unroll
  for (int et = 0; et < EPW; ++et) {
    const int e = e0 + (wv * EPW + et) * 16 + c16;
    wrow[et] = w + (size_t)(e < E ? e : E - 1) * H;
  }

  // x streams from HBM (DX steps in flight), the gate weight from L2 (D)
  constexpr int L = DX > D ? DX : D;
  static_assert(L % D == 0 && L % DX == 0, "prefetch depths must nest");
  u32x4 xreg[DX][XPT];
  u32x4 wreg[D][EPW][PQ];
  auto load_x = [&](int i, u32x4 (&dst)[XPT]) {
#pragma unroll
    for (int m = 0; m < XPT; ++m) {
      const int kk = k_lo + i * KS + xp[m] * 8;
      dst[m] = ld16(xsrc[m] + (kk < H ? kk : H - 8));
    }
  };
  auto load_w = [&](int i, u32x4 (&dst)[EPW][PQ]) {
#pragma unroll
    for (int et = 0; et < EPW; ++et)
#pragma unroll
      for (int q = 0; q < PQ; ++q) {
        const int kk = k_lo + i * KS + g * (8 * PQ) + q * 8;
        dst[et][q] = ld16(wrow[et] + (kk < H ? kk : H - 8));
      }
  };

  f32x4 acc[TT][EPW];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int et = 0; et < EPW; ++et) acc[tt][et] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int j = 0; j < DX; ++j) load_x(j, xreg[j]);
#pragma unroll
  for (int j = 0; j < D; ++j) load_w(j, wreg[j]);
  for (int i0 = 0; i0 < nss; i0 += L) {
#pragma unroll
    for (int jj = 0; jj < L; ++jj) {
      const int i = i0 + jj;
      const int jx = jj % DX, j = jj % D;
      unsigned char* slot = lds + (i & 1) * XSLOT;
#pragma unroll
      for (int m = 0; m < XPT; ++m) {
        const bool ok = xrow_ok[m] && k_lo + i * KS + xp[m] * 8 < k_hi;
        st16(slot + xr[m] * RB + ((xp[m] ^ gate_lds_swz(xr[m])) * 16),
             ok ? xreg[jx][m] : z);
      }
      lds_barrier();
      // no prefetch past the range: with few steps per range (few tokens,
      // fine hidden split) those loads would double the traffic.  Steps past
      // the range still run on zero x, and weight elements outside the range
      // (stale registers, or the next range's columns) are zeroed too, so a
      // non-finite weight there cannot turn 0 * w into NaN
#pragma unroll
      for (int q = 0; q < PQ; ++q) {
        const bool wok = k_lo + i * KS + g * (8 * PQ) + q * 8 < k_hi;
#pragma unroll
        for (int et = 0; et < EPW; ++et)
          if (!wok) wreg[j][et][q] = z;
      }
      if (i + DX < nss) load_x(i + DX, xreg[jx]);
#pragma unroll
      for (int q = 0; q < PQ; ++q) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const int r = tt * 16 + c16;
          const int p = g * PQ + q;
          Frag<uint16_t> a;
          a.v = *reinterpret_cast<const u32x4*>(slot + r * RB + ((p ^ gate_lds_swz(r)) * 16));
#pragma unroll
          for (int et = 0; et < EPW; ++et) {
            Frag<uint16_t> b;
            b.v = wreg[j][et][q];
            acc[tt][et] = mfma_step(a, b, acc[tt][et]);
          }
        }
      }
      if (i + D < nss) load_w(i + D, wreg[j]);
    }
  }
  float* out = partial + (size_t)ks * T * eps;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int et = 0; et < EPW; ++et) {
      const int e = e0 + (wv * EPW + et) * 16 + c16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + tt * 16 + g * 4 + i;
        if (t < T) out[(size_t)t * eps + e] = acc[tt][et][i];
      }
    }
}

template <int EPW, int TT, int PQ, int D, int DX = D>
__global__ __launch_bounds__(256, 1) void gate_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T,
    int H, int E, int KR, int eps, float* __restrict__ partial,
    int32_t* __restrict__ gzero, int gzero_n) {
  clear_group_totals(gzero, gzero_n);
  gate_partial_block<EPW, TT, PQ, D, DX>(blockIdx.x, blockIdx.y, blockIdx.z, x,
                                         w, T, H, E, KR, eps, partial);
}

// The same partial logits for many tokens (the same MFMAs in the same order
// per accumulator, so the same bits), with both operands staged through LDS
// by coalesced loads: 8 lanes fetch one 128-byte row segment, so a
// gate-weight segment is read once per workgroup and 64-wide k block rather
// than once per lane group and fragment.  x is loaded three blocks ahead of
// its use into two register sets (from HBM), the gate weight two blocks
// ahead into one (from L2); block b is computed from one LDS stage while
// block b+1 is written into the other.  The 2-block loop has no branches
// and its loads are unconditional (clamped to the range), which keeps the
// compiler's wait counts exact instead of draining every load each
// iteration.  Rows are XOR-swizzled in LDS by gate_lds_swz.
// Requires every range to be whole 128-element pairs of blocks
// (H % 128 == 0, KR % 128 == 0) and byte offsets below 2^32.
template <int EPW, int TT>
__global__ __launch_bounds__(512, 1) void gate_partial_lds_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T,
    int H, int E, int KR, int tiles, int xg, float* __restrict__ partial,
    int32_t* __restrict__ gzero, int gzero_n) {
  clear_group_totals(gzero, gzero_n);
  // One-dimensional grid of tiles * S workgroups; workgroup i runs on XCD
  // i % 8.  With xg = 8 / S (S dividing 8, tiles a multiple of xg) every XCD
  // serves one hidden range, so its L2 holds 1/S of the gate weight;
  // otherwise tiles vary fastest.
  int tile, ks;
  if (xg > 0) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    tile = slot * xg + xcd % xg;
    ks = xcd / xg;
  } else {
    tile = blockIdx.x % tiles;
    ks = blockIdx.x / tiles;
  }
  // 8 waves: wave wv owns tokens 16 TT (wv >> 2) + [0, 16 TT) and experts
  // 16 EPW (wv & 3) + [0, 16 EPW) of the workgroup's tile
  constexpr int EP = 64 * EPW;             // padded experts
  constexpr int TTOK = 32 * TT;            // tokens of the workgroup
  constexpr int XS = TTOK * 128;           // bytes of x in one stage
  constexpr int STG = XS + EP * 128;       // bytes of one stage
  constexpr int XPT = TTOK / 64;           // x pieces per thread and block
  constexpr int WPT = EP / 64;             // weight pieces per thread, block
  __shared__ __align__(16) unsigned char lds[2 * STG];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int t0 = tile * TTOK;
  const int k_lo = ks * KR;
  const int nb = (min(H, k_lo + KR) - k_lo) / 64;   // even, >= 2

  // this thread loads rows (tid >> 3) + 64 m, 16-byte piece tid & 7
  const int pr = tid >> 3, pc = tid & 7;
  const unsigned char* xb =
      reinterpret_cast<const unsigned char*>(x) + (size_t)k_lo * 2 + pc * 16;
  const unsigned char* wb =
      reinterpret_cast<const unsigned char*>(w) + (size_t)k_lo * 2 + pc * 16;
  const uint32_t rowb = (uint32_t)H * 2u;
  uint32_t xo[XPT], wo[WPT];
#pragma unroll
  for (int m = 0; m < XPT; ++m)
    xo[m] = (uint32_t)min(t0 + pr + 64 * m, T - 1) * rowb;
#pragma unroll
  for (int m = 0; m < WPT; ++m)
    wo[m] = (uint32_t)min(pr + 64 * m, E - 1) * rowb;
  // LDS byte offset of this thread's pieces (row pr + 64 m has pr's swizzle)
  const int dsto = pr * 128 + ((pc ^ gate_lds_swz(pr)) * 16);
  // fragment reads: row 16 j + c16 of the wave's rows, piece 2 g + q
  const int sw = gate_lds_swz(c16);
  const int frx = ((wv >> 2) * 16 * TT + c16) * 128;
  const int frw = XS + ((wv & 3) * 16 * EPW + c16) * 128;

  u32x4 xs[2][XPT], ws[WPT];
  auto load_x = [&](int b, u32x4 (&dst)[XPT]) {
    const uint32_t kb = (uint32_t)min(b, nb - 1) * 128u;
#pragma unroll
    for (int m = 0; m < XPT; ++m) dst[m] = ld16(xb + xo[m] + kb);
  };
  auto load_w = [&](int b) {
    const uint32_t kb = (uint32_t)min(b, nb - 1) * 128u;
#pragma unroll
    for (int m = 0; m < WPT; ++m) ws[m] = ld16(wb + wo[m] + kb);
  };
  auto store = [&](unsigned char* stage, const u32x4 (&src)[XPT]) {
#pragma unroll
    for (int m = 0; m < XPT; ++m) st16(stage + dsto + m * 64 * 128, src[m]);
#pragma unroll
    for (int m = 0; m < WPT; ++m)
      st16(stage + XS + dsto + m * 64 * 128, ws[m]);
  };

  f32x4 acc[TT][EPW];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int et = 0; et < EPW; ++et) acc[tt][et] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const unsigned char* stage, int q) {
    const int po = ((2 * g + q) ^ sw) * 16;
    Frag<uint16_t> b[EPW], a[TT];
#pragma unroll
    for (int et = 0; et < EPW; ++et)
      b[et].v = *reinterpret_cast<const u32x4*>(stage + frw + et * 16 * 128 + po);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
      a[tt].v = *reinterpret_cast<const u32x4*>(stage + frx + tt * 16 * 128 + po);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int et = 0; et < EPW; ++et)
        acc[tt][et] = mfma_step(a[tt], b[et], acc[tt][et]);
  };

  // block b computes stage b & 1, writes block b+1 (its weight loaded at
  // b-1, its x at b-2) into the other stage, then loads the weight of b+2
  // and the x of b+3 into the set it just stored
  load_w(0);
  load_x(0, xs[0]);
  load_x(1, xs[1]);
  store(lds, xs[0]);
  load_w(1);
  load_x(2, xs[0]);
  lds_barrier();
  for (int b = 0; b < nb; b += 2) {
    compute(lds, 0);
    store(lds + STG, xs[1]);
    load_w(b + 2);
    load_x(b + 3, xs[1]);
    compute(lds, 1);
    lds_barrier();
    compute(lds + STG, 0);
    store(lds, xs[0]);
    load_w(b + 3);
    load_x(b + 4, xs[0]);
    compute(lds + STG, 1);
    lds_barrier();
  }
  float* out = partial + (size_t)ks * T * EP;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int et = 0; et < EPW; ++et) {
      const int e = ((wv & 3) * EPW + et) * 16 + c16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + (wv >> 2) * 16 * TT + tt * 16 + g * 4 + i;
        if (t < T) out[(size_t)t * EP + e] = acc[tt][et][i];
      }
    }
}

// Sum of the S partial logits (ranges in ascending order), then the bias,
// and the top-k of every token, for 4 * WAVES tokens per workgroup (the
// tile histogram and ranks when that is 64).  The 16 lanes of a group own one
// token and lane c holds experts 64 j + 4 c + i (i < 4), so each 16-byte
// load reads four consecutive logits and a group reads 256 contiguous
// bytes; CH ranges are loaded together (clamped; the repeats are not
// added), so for S <= CH every load of a token is in flight at once.
template <int EPW, int WAVES, int CH>
__global__ __launch_bounds__(64 * WAVES) void gate_reduce_quad_kernel(
    const float* __restrict__ partial, int S, int T, int E, int k,
    const float* __restrict__ bias, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ logits_dbg,
    int32_t* __restrict__ tile_base, int32_t* __restrict__ slot_rank,
    int32_t* __restrict__ gtot) {
  constexpr int EP = 64 * EPW, ET = 4 * EPW;
  constexpr int NT = 64 * WAVES, TOK = 4 * WAVES;
  constexpr bool HIST = TOK == 64;
  __shared__ unsigned long long tile_bits[HIST ? EP : 1];
  __shared__ int tile_sel[HIST ? 64 * MOE_MAX_TOPK : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int t0 = blockIdx.x * TOK;
  const int tl = wv * 4 + g;
  const int t = t0 + tl;
  const int tc = t < T ? t : T - 1;
  if constexpr (HIST) {
    for (int e = tid; e < EP; e += NT) tile_bits[e] = 0ull;
    __syncthreads();
  }
  const float* row = partial + (size_t)tc * EP + 4 * c16;
  const size_t rs = (size_t)T * EP;        // stride between ranges
  float v[ET];
  auto load = [&](int q0, f32x4 (&u)[CH][EPW]) {
#pragma unroll
    for (int b = 0; b < CH; ++b) {
      const int q = q0 + b < S ? q0 + b : S - 1;
#pragma unroll
      for (int j = 0; j < EPW; ++j)
        u[b][j] = __builtin_bit_cast(f32x4, ld16(row + q * rs + 64 * j));
    }
  };
  {
    f32x4 u[CH][EPW];
    load(0, u);
#pragma unroll
    for (int j = 0; j < EPW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * j + i] = u[0][j][i];
#pragma unroll
    for (int b = 1; b < CH; ++b)
      if (b < S) {
#pragma unroll
        for (int j = 0; j < EPW; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * j + i] += u[b][j][i];
      }
  }
  for (int q0 = CH; q0 < S; q0 += CH) {
    f32x4 u[CH][EPW];
    load(q0, u);
#pragma unroll
    for (int b = 0; b < CH; ++b)
      if (q0 + b < S) {
#pragma unroll
        for (int j = 0; j < EPW; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * j + i] += u[b][j][i];
      }
  }
#pragma unroll
  for (int et = 0; et < ET; ++et) {
    const int e = topk_expert<true>(et, c16);
    v[et] += (bias != nullptr && e < E) ? bias[e] : 0.0f;
    if (logits_dbg != nullptr && t < T && e < E)
      logits_dbg[(size_t)t * E + e] = v[et];
  }
  if constexpr (HIST)
    topk_select_write<ET, true, (WAVES < 16 || ET <= 16)>(
        v, t, T, E, k, topk_idx, topk_w, tile_bits, tile_sel, tl);
  else
    topk_select_write<ET, true, (WAVES < 16 || ET <= 16)>(
        v, t, T, E, k, topk_idx, topk_w);
  if constexpr (HIST) {
    __syncthreads();
    for (int e = tid; e < E; e += NT) {
      const int c = __popcll(tile_bits[e]);
      tile_base[(size_t)blockIdx.x * E + e] = c;
      if (gtot != nullptr && c != 0)
        atomicAdd(&gtot[(size_t)(blockIdx.x / kScanGroup) * E + e], c);
    }
    const int n = min(64, T - t0) * k;
    for (int q = tid; q < n; q += NT) {
      const int tq = q / k, j = q - tq * k;
      const int e = tile_sel[tq * MOE_MAX_TOPK + j];
      slot_rank[(size_t)t0 * k + q] =
          __popcll(tile_bits[e] & ((1ull << tq) - 1ull));
    }
  }
}

template <typename XT, int ET>
__global__ __launch_bounds__(256) void gate_topk_ksplit_kernel(
    const XT* __restrict__ x, const XT* __restrict__ w,
    const float* __restrict__ bias, int T, int H, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits_dbg) {
  // k steps in flight per wave: a workgroup per 16 tokens leaves one per
  // CU, so each must keep enough of its x stream in flight on its own
  // (4 steps, 16 KB per CU, held the stream to ~2 TB/s)
  constexpr int U = sizeof(XT) == 2 ? 16 : 8;
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
      frag_load<XT>(a[u], xrow + kk, arow_ok && kok, false);
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
// With gtot, each tile's counts are also added to its group's totals (the
// parallel scan's input; cleared earlier in the same call).
__global__ __launch_bounds__(256) void tile_histogram_kernel(
    const int32_t* __restrict__ topk_idx, int T, int k, int E,
    int32_t* __restrict__ tile_base, int32_t* __restrict__ slot_rank,
    int32_t* __restrict__ gtot) {
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
  for (int e = tid; e < E; e += 256) {
    const int c = __popcll(bits[e]);
    tile_base[(size_t)tile * E + e] = c;
    if (gtot != nullptr && c != 0)
      atomicAdd(&gtot[(size_t)(tile / kScanGroup) * E + e], c);
  }
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
// contiguous run of tiles of expert e.  Pass 1 sums the runs (32 loads in
// flight per thread), an LDS pass and a shuffle scan give each run's start
// and the padded expert offsets, pass 2 overwrites every tile count with the
// first row of that (tile, expert) run: offsets[e] + tokens of e in earlier
// tiles.  Runs of up to 32 tiles stay in registers between the passes.
__global__ __launch_bounds__(1024) void expert_scan_kernel(
    int32_t* __restrict__ tile_base, int ntiles, int E, int pad,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  constexpr int B = 32;
  __shared__ int part[1024];
  __shared__ int scan[1024];
  const int tid = threadIdx.x;
  int parts = 1024 / E;
  if (parts > ntiles) parts = ntiles;
  const int e = tid % E, p = tid / E;
  const bool active = p < parts;
  const int lo = active ? (int)((long long)p * ntiles / parts) : 0;
  const int hi = active ? (int)((long long)(p + 1) * ntiles / parts) : 0;

  // loads are unconditional (clamped row) so a batch is in flight together
  int v[B];
  int sum = 0;
  const int last = hi > lo ? hi - 1 : 0;
  for (int b0 = lo; b0 < hi; b0 += B) {
#pragma unroll
    for (int u = 0; u < B; ++u)
      v[u] = tile_base[(size_t)min(b0 + u, last) * E + e];
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (b0 + u < hi) sum += v[u];
  }
  if (active) part[p * E + e] = sum;
  __syncthreads();
  int padded = 0;
  if (tid < E) {
    int run = 0;
    for (int q = 0; q < parts; ++q) {
      const int c = part[q * E + tid];
      part[q * E + tid] = run;
      run += c;
    }
    counts[tid] = run;
    padded = (run + pad - 1) / pad * pad;
  }
  // inclusive scan of the padded counts: within each wave by shuffles,
  // then across the 16 wave totals
  const int ln = tid & 63, wid = tid >> 6;
  int incl = padded;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (ln >= off) incl += o;
  }
  __shared__ int wsum[16];
  if (ln == 63) wsum[wid] = incl;
  __syncthreads();
  int before = 0;
  for (int q = 0; q < wid; ++q) before += wsum[q];
  scan[tid] = incl + before;
  __syncthreads();
  if (tid < E) offsets[tid + 1] = scan[tid];
  if (tid == 0) offsets[0] = 0;
  if (active) {
    int run = part[p * E + e] + (e == 0 ? 0 : scan[e - 1]);
    const bool kept = hi - lo <= B;     // the single batch is still in v
    for (int b0 = lo; b0 < hi; b0 += B) {
      if (!kept) {
#pragma unroll
        for (int u = 0; u < B; ++u)
          v[u] = tile_base[(size_t)min(b0 + u, last) * E + e];
      }
#pragma unroll
      for (int u = 0; u < B; ++u) {
        if (b0 + u < hi) {
          tile_base[(size_t)(b0 + u) * E + e] = run;
          run += v[u];
        }
      }
    }
  }
}

// Parallel form of the scan, one workgroup per group of kScanGroup tiles,
// from the per-group expert totals the histogram producers accumulated:
// every workgroup adds the totals of all groups (experts' counts) and of the
// groups before its own, scans the padded counts over the experts (the
// offsets; workgroup 0 stores counts and offsets) and turns its tiles'
// counts into first rows.  No workgroup reads another group's tiles.
template <int PER>   // experts per thread: E <= 256 * PER
__global__ __launch_bounds__(256) void expert_scan_groups_kernel(
    int32_t* __restrict__ tile_base, int ntiles, int E, int pad,
    const int32_t* __restrict__ gtot, int ngroups,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  constexpr int B = 16;                        // loads in flight
  __shared__ int wsum[4];
  const int tid = threadIdx.x, g = blockIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  int tot[PER], pre[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    tot[i] = 0;
    pre[i] = 0;
  }
  // thread tid owns experts tid * PER + i (consecutive, for the scan)
  for (int q0 = 0; q0 < ngroups; q0 += B) {
    int v[B][PER];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int q = min(q0 + b, ngroups - 1);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = tid * PER + i;
        v[b][i] = gtot[(size_t)q * E + (e < E ? e : E - 1)];
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int q = q0 + b;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if (q < ngroups) tot[i] += v[b][i];
        if (q < g) pre[i] += v[b][i];
      }
    }
  }
  int padded[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid * PER + i;
    padded[i] = e < E ? (tot[i] + pad - 1) / pad * pad : 0;
    sum += padded[i];
  }
  // exclusive scan of the thread sums: within each wave, then the 4 waves
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int q = 0; q < wv; ++q) run += wsum[q];
  int first[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    first[i] = run;
    run += padded[i];
  }
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid * PER + i;
      if (e < E) {
        counts[e] = tot[i];
        offsets[e] = first[i];
      }
    }
    if (tid == 255) offsets[E] = run;
  }
  // this group's tiles: first row = offsets[e] + earlier groups + earlier
  // tiles of the group
  const int t0 = g * kScanGroup;
  const int nt = min(kScanGroup, ntiles - t0);
  int c[kScanGroup][PER];
#pragma unroll
  for (int j = 0; j < kScanGroup; ++j)
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid * PER + i;
      c[j][i] = tile_base[(size_t)(t0 + min(j, nt - 1)) * E +
                          (e < E ? e : E - 1)];
    }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid * PER + i;
    int base = first[i] + pre[i];
#pragma unroll
    for (int j = 0; j < kScanGroup; ++j) {
      if (j < nt && e < E) {
        tile_base[(size_t)(t0 + j) * E + e] = base;
        base += c[j][i];
      }
    }
  }
}

// ------------------------------------------------------------------ small batches

// Histogram, padded scan, first rows and ranks of all T <= kSmallPlanT
// tokens in one workgroup of NT threads (the same results as
// tile_histogram_kernel followed by expert_scan_kernel).  bits: LDS
// [ceil(T/64) * E] 64-bit tile ballots; ecnt: LDS [E].
template <int NT>
__device__ void small_plan(const int32_t* __restrict__ topk_idx, int T, int k,
                           int E, int pad, int32_t* __restrict__ counts,
                           int32_t* __restrict__ offsets,
                           int32_t* __restrict__ tile_base,
                           int32_t* __restrict__ slot_rank,
                           unsigned long long* bits, int* ecnt) {
  const int tid = threadIdx.x;
  const int nt = (T + 63) / 64;
  for (int i = tid; i < nt * E; i += NT) bits[i] = 0ull;
  __syncthreads();
  const int n = T * k;
  for (int p = tid; p < n; p += NT) {
    const int e = topk_idx[p];
    const int t = p / k;
    if (e >= 0 && e < E) atomicOr(&bits[(t >> 6) * E + e], 1ull << (t & 63));
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    int c = 0;
    for (int q = 0; q < nt; ++q) c += __popcll(bits[q * E + e]);
    counts[e] = c;
    ecnt[e] = (c + pad - 1) / pad * pad;
  }
  __syncthreads();
  if (tid < 64) {
    // exclusive scan of the padded counts (also the offsets)
    const int total =
        wave_exclusive_scan<MOE_MAX_EXPERTS / 64>(ecnt, E, offsets);
    if (tid == 0) offsets[E] = total;
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    int run = ecnt[e];
    for (int q = 0; q < nt; ++q) {
      tile_base[(size_t)q * E + e] = run;
      run += __popcll(bits[q * E + e]);
    }
  }
  for (int p = tid; p < n; p += NT) {
    const int e = topk_idx[p];
    const int t = p / k;
    int r = -1;
    if (e >= 0 && e < E)
      r = __popcll(bits[(t >> 6) * E + e] & ((1ull << (t & 63)) - 1ull));
    slot_rank[p] = r;
  }
}

// moe_plan for few tokens: one workgroup instead of histogram + scan.
__global__ __launch_bounds__(512) void plan_small_kernel(
    const int32_t* __restrict__ topk_idx, int T, int k, int E, int pad,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ tile_base, int32_t* __restrict__ slot_rank) {
  __shared__ unsigned long long bits[(kSmallPlanT / 64) * MOE_MAX_EXPERTS];
  __shared__ int ecnt[MOE_MAX_EXPERTS];
  small_plan<512>(topk_idx, T, k, E, pad, counts, offsets, tile_base,
                  slot_rank, bits, ecnt);
}

// Maximum over the 64 lanes of a wave (result uniform): 16-lane DPP maxima,
// then the four row maxima read into scalar registers.
__device__ __forceinline__ unsigned long long max64_u64(unsigned long long v) {
  v = max16_u64(v);
  unsigned long long m = 0ull;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 16 * r);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 16 * r);
    const unsigned long long x = ((unsigned long long)hi << 32) | lo;
    m = x > m ? x : m;
  }
  return m;
}

// Reduction of the split gate for few tokens: a workgroup of RW waves (8 in
// gate_reduce_small_kernel) covers TPW tokens with WPT = RW / TPW waves each.  Wave p of a token adds the
// ranges p, p + WPT, ... in ascending order, each lane holding C4 groups of
// 4 consecutive experts (16-byte loads across the whole logit row); the
// token's first wave adds its WPT wave sums in wave order (fixed order: the
// logits do not depend on timing) and selects the top-k with all 64 lanes
// (same 64-bit keys and tie-break as topk_select_write).  The plan follows
// as plan_small_kernel: a separate launch costs less than having the last
// workgroup plan after device-scope release/acquire fences in every one.
// Workgroup blk of RW waves (TPW tokens of RW / TPW waves each).
template <int C4, int TPW, int RW>
__device__ __forceinline__ void gate_reduce_small_block(
    int blk, const float* __restrict__ partial, int S, int EPS, int T, int E,
    int k, const float* __restrict__ bias, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ logits_dbg) {
  constexpr int B = 8;                          // ranges in flight
  constexpr int WPT = RW / TPW;                 // waves per token
  __shared__ f32x4 red[RW * 64 * C4];           // wave sums
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int tk = wv / WPT, part = wv - tk * WPT;
  const int t = blk * TPW + tk;
  const bool live = t < T;
  const int tc = live ? t : T - 1;
  const int nc4 = EPS / 4;                      // 16-byte groups of a row

  f32x4 v[C4];
#pragma unroll
  for (int c = 0; c < C4; ++c) v[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int q0 = part; q0 < S; q0 += B * WPT) {
    f32x4 u[B][C4];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int q = q0 + b * WPT < S ? q0 + b * WPT : q0;
      const f32x4* pq = (const f32x4*)(partial + ((size_t)q * T + tc) * EPS);
#pragma unroll
      for (int c = 0; c < C4; ++c) {
        const int ci = lane + 64 * c;
        u[b][c] = pq[ci < nc4 ? ci : 0];
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b)
      if (q0 + b * WPT < S) {
#pragma unroll
        for (int c = 0; c < C4; ++c) v[c] += u[b][c];
      }
  }
#pragma unroll
  for (int c = 0; c < C4; ++c) red[(wv * C4 + c) * 64 + lane] = v[c];
  __syncthreads();
  if (part == 0 && live) {
    unsigned long long key[C4 * 4];
#pragma unroll
    for (int c = 0; c < C4; ++c) {
      f32x4 a = red[(wv * C4 + c) * 64 + lane];
      for (int w = 1; w < WPT; ++w) a += red[((wv + w) * C4 + c) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * (lane + 64 * c) + i;
        const bool ok = e < E && lane + 64 * c < nc4;
        const float l = a[i] + ((bias != nullptr && ok) ? bias[e] : 0.0f);
        if (logits_dbg != nullptr && ok) logits_dbg[(size_t)t * E + e] = l;
        key[c * 4 + i] = ok ? ((unsigned long long)f32_order_key(l) << 32) |
                                  (0xffffffffu - (uint32_t)e)
                            : 0ull;
      }
    }
    // this lane's keys in descending order (odd-even transposition), so a
    // round's candidate is key[0] and the winning lane shifts its list
    constexpr int NK = C4 * 4;
#pragma unroll
    for (int r = 0; r < NK; ++r)
#pragma unroll
      for (int i = r & 1; i + 1 < NK; i += 2) {
        const unsigned long long hi = key[i] > key[i + 1] ? key[i] : key[i + 1];
        const unsigned long long lo = key[i] > key[i + 1] ? key[i + 1] : key[i];
        key[i] = hi;
        key[i + 1] = lo;
      }
    // k rounds of a 64-lane max; lane j keeps the j-th choice
    int my_e = 0;
    uint32_t my_key = 0u, top_key = 0u;
    for (int j = 0; j < k; ++j) {
      const unsigned long long best = max64_u64(key[0]);
      const uint32_t blo = (uint32_t)best;
      const bool win = (uint32_t)key[0] == blo;
#pragma unroll
      for (int i = 0; i + 1 < NK; ++i) key[i] = win ? key[i + 1] : key[i];
      key[NK - 1] = win ? 0ull : key[NK - 1];
      if (lane == j) {
        my_e = (int)(0xffffffffu - blo);
        my_key = (uint32_t)(best >> 32);
      }
      if (j == 0) top_key = (uint32_t)(best >> 32);
    }
    // weights exp(l_j - l_0) / sum over the chosen, the sum in choice order
    const float ex = lane < k ? expf(f32_from_order_key(my_key) -
                                     f32_from_order_key(top_key))
                              : 0.0f;
    float den = 0.0f;
    for (int j = 0; j < k; ++j)
      den += __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(ex), j));
    if (lane < k) {
      topk_idx[(size_t)t * k + lane] = my_e;
      topk_w[(size_t)t * k + lane] = ex / den;
    }
  }
}

template <int C4, int TPW>
__global__ __launch_bounds__(512) void gate_reduce_small_kernel(
    const float* __restrict__ partial, int S, int EPS, int T, int E, int k,
    const float* __restrict__ bias, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ logits_dbg) {
  gate_reduce_small_block<C4, TPW, 8>(blockIdx.x, partial, S, EPS, T, E, k,
                                      bias, topk_idx, topk_w, logits_dbg);
}


// ------------------------------------------------------------------ one launch

// Arrival counters of the one-launch path's grid-wide waits, per GPU: [0]
// all arrivals, [32 (1 + x)] the arrivals of the workgroups on XCD x.  They
// only grow; the host passes the value of [0] at the start of each call.
__device__ __align__(256) unsigned long long g_one_launch_bar[9 * 32];

// Every workgroup of a grid of G (a multiple of 8; workgroup i runs on XCD
// i % 8) waits here until all G have arrived for the n-th time in this call.
// What a workgroup wrote before the wait is visible to every workgroup after
// it: each arrival follows a device-scope release, the last arrival of an
// XCD acquires its XCD's arrivals and adds them to the global count with a
// release, and every workgroup acquires once it sees the count complete.
// The spin is bounded (2^20 polls, on the order of a second): calls that
// overlap on one GPU, which the entry point rules out, could then give wrong
// results but cannot hang the GPU.
__device__ void one_launch_wait(int n, int G, unsigned long long gbase) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long nx = (unsigned long long)(G / 8);
    unsigned long long* xc = &g_one_launch_bar[32 * (1 + (blockIdx.x & 7))];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned long long t = __hip_atomic_fetch_add(
        xc, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t + 1 == gbase / 8 + (unsigned long long)n * nx) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_fetch_add(&g_one_launch_bar[0], nx, __ATOMIC_RELEASE,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
    const unsigned long long target = gbase + (unsigned long long)n * G;
    for (long i = 0; i < (1l << 20); ++i) {
      if (__hip_atomic_load(&g_one_launch_bar[0], __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT) >= target)
        break;
      __builtin_amdgcn_s_sleep(2);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// Gate, top-k, plan and scatter of T <= 256 bf16 tokens in one launch: the
// split gate's partial logits (workgroups as gate_partial_kernel's grid of
// tiles x ranges x expert groups), a grid-wide wait, the reduction and top-k
// of one token per workgroup (4 waves share its ranges), a second wait, then
// every workgroup rebuilds the plan in LDS and runs its share of the scatter
// blocks and the padding fill, as plan_dispatch_small_kernel does.
template <int C4, int KMAX, int MODE>
__global__ __launch_bounds__(256) void route_dispatch_one_launch_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const float* __restrict__ bias, int T, int H, int E, int k, int pad,
    int KR, int S, int tiles, int eg, float* __restrict__ part,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits_dbg, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, unsigned char* __restrict__ rows,
    long long capacity, float* __restrict__ row_scales,
    int32_t* __restrict__ row_src, int32_t* __restrict__ tok_row,
    int tok_blocks, int hsplit, unsigned long long gbase) {
  const int G = gridDim.x, wg = blockIdx.x;
  const int eps = 64 * eg;
  const int ngate = tiles * S * eg;
  for (int b = wg; b < ngate; b += G) {
    gate_partial_block<1, 2, 2, 2>(b % tiles, (b / tiles) % S,
                                   b / (tiles * S), x, w, T, H, E, KR, eps,
                                   part);
    __syncthreads();
  }
  one_launch_wait(1, G, gbase);
  for (int t = wg; t < T; t += G) {
    gate_reduce_small_block<C4, 1, 4>(t, part, S, eps, T, E, k, bias,
                                      topk_idx, topk_w, logits_dbg);
    __syncthreads();
  }
  one_launch_wait(2, G, gbase);
  extern __shared__ unsigned long long plan_lds[];
  LocalPlan p = local_plan_arrays(plan_lds, T, E);
  local_plan(topk_idx, T, k, E, pad, p.bits, p.base, p.cnt, p.off);
  const int nblk = tok_blocks + kDispatchFillBlocks;
  for (int b = wg; b < nblk; b += G)
    plan_dispatch_block<KMAX, MODE, 1>(
        b, reinterpret_cast<const unsigned char*>(x), 2, T, H, topk_idx, k, E,
        counts, offsets, rows, capacity, row_scales, row_src, tok_row,
        tok_blocks, hsplit, p);
}

// ------------------------------------------------------------------ launchers

// What remains of moe_route after the gate kernels: the whole plan, the
// one-workgroup scan (tile counts and ranks written by the gate's
// epilogue), the tile histogram and the parallel scan, or the parallel scan
// alone (histogram fused into the reduction).
enum {
  kRouteNeedPlan = 0,
  kRouteNeedScan = 1,
  kRouteNeedGroupHist = 2,
  kRouteNeedGroupScan = 3
};

// Per-group expert totals of the parallel scan, after the partial logits.
static int32_t* ws_groups(void* ws, int T, int E, int k) {
  return (int32_t*)((unsigned char*)ws + ws_tile_bytes(T, E) +
                    ws_rank_bytes(T, k) + ws_partial_bytes(T, E));
}

template <typename XT>
static hipError_t launch_gate_typed(const XT* x, const XT* w, const float* bias,
                                    int T, int H, int E, int k,
                                    int32_t* idx, float* tw, float* dbg,
                                    int32_t* tb, int32_t* sr, int* stage,
                                    hipStream_t s) {
  *stage = kRouteNeedPlan;
  const int et = (E + 15) / 16;
  // few experts: the k-split single pass, except for many bf16 tokens,
  // where the LDS-staged split gate streams x faster
  const bool few_lds = sizeof(XT) == 2 && T >= 4096 && H % 128 == 0;
  if (et <= 2 && !few_lds) {
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
  if constexpr (sizeof(XT) == 2) {
    if (E > kGateWideE) {
      // More than 512 experts (T <= kSplitMaxT, checked by the API):
      // partial logits over hidden ranges in expert groups of 256 (also
      // with a single range), then the top-k of each token over all 64
      // lanes of a wave (16 logits per lane at 1024 experts) and the plan
      // kernels.
      const int epw = gate_epw(E);                 // 12 or 16
      const int eg = epw / 4;
      const int tiles = (T + 63) / 64;
      int S = (256 + tiles * eg - 1) / (tiles * eg);
      S = max(1, min(S, min(split_max(T), (H + 63) / 64)));
      const int KR = ((H + S - 1) / S + 63) / 64 * 64;
      S = (H + KR - 1) / KR;
      float* part = (float*)((unsigned char*)sr + ws_rank_bytes(T, k));
      hipLaunchKernelGGL((gate_partial_kernel<4, 4, 2, 4>),
                         dim3(tiles, S, eg), dim3(256), 0, s, x, w, T, H, E,
                         KR, 64 * epw, part, nullptr, 0);
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      const int EPS = 64 * epw;
      const bool few = T <= kSmallPlanT;   // one token per workgroup
      const dim3 rgrid(few ? T : (T + 7) / 8);
#define MOE_GATE_RS(C4V, TPWV)                                                \
  hipLaunchKernelGGL((gate_reduce_small_kernel<C4V, TPWV>), rgrid, dim3(512), \
                     0, s, part, S, EPS, T, E, k, bias, idx, tw, dbg)
      if (epw == 12) {
        if (few) MOE_GATE_RS(3, 1);
        else MOE_GATE_RS(3, 8);
      } else {
        if (few) MOE_GATE_RS(4, 1);
        else MOE_GATE_RS(4, 8);
      }
#undef MOE_GATE_RS
      *stage = kRouteNeedPlan;
      return hipGetLastError();
    }
    // Narrow gate (the whole weight under 1 MiB, e.g. H = 768 with 384
    // experts): 32-token one-pass workgroups that each stream the whole
    // weight from L2 beat the split gate, whose partial logits cost more
    // than the GEMM itself; then the tile histogram and the parallel scan.
    // Measured faster from 4096 to 32768 tokens with 64 to 512 experts
    // (route at 8192 x 768 x 384: 40.5 -> 29 us); at 65536 tokens, with a
    // 1 MiB weight, or with fewer experts (padded to 128 here) the split gate
    // stays ahead.
    const int en = (E + 127) / 128;
    if (T >= 4096 && T <= 32768 && E >= 64 && E <= 512 && H % 64 == 0 &&
        (size_t)E * H * 2 < ((size_t)1 << 20)) {
      int32_t* gz = (int32_t*)((unsigned char*)sr + ws_rank_bytes(T, k) +
                               ws_partial_bytes(T, E));
      const int gzn = num_groups(T) * E;
      const dim3 ngrid((T + 31) / 32);
#define MOE_GATE_NARROW(EPWV)                                               \
  hipLaunchKernelGGL((gate_topk_narrow_kernel<EPWV>), ngrid, dim3(512), 0, \
                     s, x, w, bias, T, H, E, k, idx, tw, dbg, gz, gzn)
      if (en == 1) MOE_GATE_NARROW(1);
      else if (en == 2) MOE_GATE_NARROW(2);
      else if (en == 3) MOE_GATE_NARROW(3);
      else MOE_GATE_NARROW(4);
#undef MOE_GATE_NARROW
      *stage = kRouteNeedGroupHist;
      return hipGetLastError();
    }
    const int epw = gate_epw(E);
    // Split the hidden dimension so the partial GEMM runs about 256
    // workgroups; with a full chip that beats the fused single pass even
    // at 16K tokens.  Below 4096 tokens (gate_partial_kernel) workgroups
    // also split the experts: up to kSmallPlanT tokens 32-token tiles and
    // one group of 64 experts per workgroup, ~224 workgroups; above that
    // 64-token tiles, 64 experts per workgroup up to 2048 tokens and 128
    // beyond, 4 or 8 hidden ranges (8 while that stays within ~800
    // workgroups).  Less gate weight per workgroup and fewer ranges to add
    // measured 1.2-2.3x faster than whole expert rows per workgroup.
    // From 4096 tokens the LDS-staged kernel takes 128-token tiles with
    // coalesced loads of both operands; it needs hidden ranges of whole
    // 128-element block pairs and 32-bit byte offsets.  Otherwise
    // gate_partial_kernel, whose lane groups load gate-weight fragments
    // directly (128-token tiles at 8K tokens and up halve that traffic).
    const bool lds_gate = T >= 4096 && H % 128 == 0 &&
                          (epw <= 4 || epw == 6) &&
                          (size_t)T * H * 2 <= 0xffffffffu &&
                          (size_t)E * H * 2 <= 0xffffffffu;
    // LDS-staged gate: 64-token tiles up to 8192 tokens (more workgroups
    // for a smaller hidden split, so fewer partials), 128-token tiles above
    const bool small = T <= kSmallPlanT;
    const bool mid = !lds_gate && !small && T < 4096;
    const int TT = lds_gate ? (T > 8192 ? 8 : 4)
                   : small ? 2 : mid ? 4
                   : (epw <= 4 && T >= 8192) ? 8 : 4;
    const int tiles = (T + 16 * TT - 1) / (16 * TT);
    // 64-expert tiles per workgroup, and expert groups
    const int epg = (mid && T > 2048 && epw % 2 == 0) ? 2 : 1;
    const int eg = (small || mid) ? epw / epg : 1;
    const int kq = lds_gate ? 128 : 64;    // range granularity
    int S;
    if (mid) {
      S = tiles * eg * 8 <= 800 ? 8 : 4;
    } else if (lds_gate) {
      // one workgroup per CU: the split S of 2..4 with the least work per
      // CU, rounds(S) / S with rounds = ceil(tiles * S / 256), the fewer
      // ranges on a tie (measured best at 8K-32K tokens; 2 at 16384)
      S = 2;
      for (int c = 3; c <= 4; ++c) {
        const long long rc = ((long long)tiles * c + 255) / 256;
        const long long rs = ((long long)tiles * S + 255) / 256;
        if (rc * S < rs * c) S = c;
      }
    } else {
      const int target = small ? 224 : 256;
      S = (target + tiles * eg - 1) / (tiles * eg);
    }
    S = min(S, min(split_max(T), (H + kq - 1) / kq));
    if (S > 1) {
      const int KR = ((H + S - 1) / S + kq - 1) / kq * kq;
      S = (H + KR - 1) / KR;
      float* part = (float*)((unsigned char*)sr + ws_rank_bytes(T, k));
      // group totals of the parallel scan, cleared by the partial gate
      int32_t* gz = small ? nullptr
                          : (int32_t*)((unsigned char*)part +
                                       ws_partial_bytes(T, E));
      const int gzn = small ? 0 : num_groups(T) * E;
      const dim3 pgrid(tiles, S, eg);
#define MOE_GATE_PART(EPWV, TTV, DV)                                           \
  hipLaunchKernelGGL((gate_partial_kernel<EPWV, TTV, 2, DV>), pgrid,          \
                     dim3(256), 0, s, x, w, T, H, E, KR, 64 * EPWV, part, gz, \
                     gzn)
#define MOE_GATE_PART_X(EPWV, TTV, DV, DXV)                                    \
  hipLaunchKernelGGL((gate_partial_kernel<EPWV, TTV, 2, DV, DXV>), pgrid,     \
                     dim3(256), 0, s, x, w, T, H, E, KR, 64 * EPWV, part, gz, \
                     gzn)
#define MOE_GATE_PART_E(TTV)                                                   \
  do {                                                                         \
    if (epw == 1) MOE_GATE_PART(1, TTV, 4);                                    \
    else if (epw == 2) MOE_GATE_PART(2, TTV, 4);                               \
    else if (epw == 4) MOE_GATE_PART(4, TTV, 4);                               \
    else if (epw == 6) MOE_GATE_PART(6, TTV, 3);                               \
    else MOE_GATE_PART(8, TTV, 2);                                             \
  } while (0)
      const int xg = (8 % S == 0 && tiles % (8 / S) == 0) ? 8 / S : 0;
#define MOE_GATE_LDS_T(EPWV, TTV)                                              \
  hipLaunchKernelGGL((gate_partial_lds_kernel<EPWV, TTV>), dim3(tiles * S),   \
                     dim3(512), 0, s, x, w, T, H, E, KR, tiles, xg, part, gz, \
                     gzn)
#define MOE_GATE_LDS(EPWV)                                                     \
  do {                                                                         \
    if (TT == 8) MOE_GATE_LDS_T(EPWV, 4);                                      \
    else MOE_GATE_LDS_T(EPWV, 2);                                              \
  } while (0)
      if (small) {
        hipLaunchKernelGGL((gate_partial_kernel<1, 2, 2, 2>), pgrid,
                           dim3(256), 0, s, x, w, T, H, E, KR, 64 * epw, part,
                           gz, gzn);
      } else if (mid) {
        if (epg == 1)
          hipLaunchKernelGGL((gate_partial_kernel<1, 4, 2, 2>), pgrid,
                             dim3(256), 0, s, x, w, T, H, E, KR, 64 * epw,
                             part, gz, gzn);
        else
          hipLaunchKernelGGL((gate_partial_kernel<2, 4, 2, 2>), pgrid,
                             dim3(256), 0, s, x, w, T, H, E, KR, 64 * epw,
                             part, gz, gzn);
      } else if (lds_gate) {
        if (epw == 1) MOE_GATE_LDS(1);
        else if (epw == 2) MOE_GATE_LDS(2);
        else if (epw == 4) MOE_GATE_LDS(4);
        else MOE_GATE_LDS(6);
      } else if (TT == 8) {
        if (epw == 1) MOE_GATE_PART(1, 8, 3);
        else if (epw == 2) MOE_GATE_PART(2, 8, 3);
        else MOE_GATE_PART_X(4, 8, 2, 4);   // x 4 steps ahead: +5%
      } else {
        MOE_GATE_PART_E(4);
      }
#undef MOE_GATE_LDS
#undef MOE_GATE_LDS_T
#undef MOE_GATE_PART_E
#undef MOE_GATE_PART_X
#undef MOE_GATE_PART
      hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      const int EPS = 64 * epw;
      if (small) {
        // reduction and top-k with one token per workgroup (its 8 waves
        // share the ranges), then plan_small_kernel
        const dim3 rgrid(T);
        if (epw <= 4)
          hipLaunchKernelGGL((gate_reduce_small_kernel<1, 1>), rgrid,
                             dim3(512), 0, s, part, S, EPS, T, E, k, bias,
                             idx, tw, dbg);
        else
          hipLaunchKernelGGL((gate_reduce_small_kernel<2, 1>), rgrid,
                             dim3(512), 0, s, part, S, EPS, T, E, k, bias,
                             idx, tw, dbg);
        *stage = kRouteNeedPlan;
        return hipGetLastError();
      }
      // reduction: 64-token workgroups that also build the tile histogram
      // once they alone fill every CU (its top-k is VALU-bound, so fewer
      // workgroups leave CUs idle), otherwise 16-token workgroups and a
      // separate histogram pass; all ranges of a token in flight at once up
      // to S = 4 (2 for the widest expert counts)
      const bool fuse = (T + 63) / 64 >= 256;
      const dim3 rgrid(fuse ? (T + 63) / 64 : (T + 15) / 16);
      const int ch = S == 2 ? 2 : S == 3 ? 3 : epw >= 6 ? 2 : 4;
#define MOE_GATE_RQ(EPWV, WV, CHV)                                             \
  hipLaunchKernelGGL((gate_reduce_quad_kernel<EPWV, WV, CHV>), rgrid,         \
                     dim3(64 * WV), 0, s, part, S, T, E, k, bias, idx, tw,    \
                     dbg, tb, sr, fuse ? gz : nullptr)
#define MOE_GATE_RQ_W(EPWV, CHV)                                               \
  do {                                                                         \
    if (fuse) MOE_GATE_RQ(EPWV, 16, CHV);                                      \
    else MOE_GATE_RQ(EPWV, 4, CHV);                                            \
  } while (0)
#define MOE_GATE_RQ_E(EPWV)                                                    \
  do {                                                                         \
    if (ch == 2) MOE_GATE_RQ_W(EPWV, 2);                                       \
    else if (ch == 3) MOE_GATE_RQ_W(EPWV, 3);                                  \
    else MOE_GATE_RQ_W(EPWV, 4);                                               \
  } while (0)
      if (epw == 1) MOE_GATE_RQ_E(1);
      else if (epw == 2) MOE_GATE_RQ_E(2);
      else if (epw == 4) MOE_GATE_RQ_E(4);
      else if (epw == 6) {
        if (ch == 3) MOE_GATE_RQ_W(6, 3);
        else MOE_GATE_RQ_W(6, 2);
      } else {
        if (ch == 3) MOE_GATE_RQ_W(8, 3);
        else MOE_GATE_RQ_W(8, 2);
      }
#undef MOE_GATE_RQ_E
#undef MOE_GATE_RQ_W
#undef MOE_GATE_RQ
      *stage = fuse ? kRouteNeedGroupScan : kRouteNeedGroupHist;
      return hipGetLastError();
    }
#define MOE_GATE_V2(EPWV, PQV, DV)                                         \
  hipLaunchKernelGGL((gate_topk_v2_kernel<EPWV, PQV, DV>), grid, dim3(256), \
                     0, s, x, w, bias, T, H, E, k, idx, tw, dbg, tb, sr)
    if (epw == 1) MOE_GATE_V2(1, 2, 4);
    else if (epw == 2) MOE_GATE_V2(2, 2, 4);
    else if (epw == 4) MOE_GATE_V2(4, 2, 4);
    else if (epw == 6) MOE_GATE_V2(6, 2, 3);
    else MOE_GATE_V2(8, 2, 2);
#undef MOE_GATE_V2
    *stage = kRouteNeedScan;
    return hipGetLastError();
  }
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

hipError_t launch_plan(const int32_t* topk_idx, int T, int k, int E, int pad,
                       int32_t* counts, int32_t* offsets, void* workspace,
                       hipStream_t s);

static hipError_t launch_scan(int32_t* tile_base, int nt, int E, int pad,
                              int32_t* counts, int32_t* offsets,
                              hipStream_t s) {
  hipLaunchKernelGGL(expert_scan_kernel, dim3(1), dim3(1024), 0, s, tile_base,
                     nt, E, pad, counts, offsets);
  return hipGetLastError();
}

// The rest of the plan after the gate kernels, by what they left to do.
static hipError_t finish_plan(int stage, const int32_t* topk_idx, int T,
                              int k, int E, int pad, int32_t* counts,
                              int32_t* offsets, void* workspace,
                              hipStream_t s) {
  int32_t* tile_base = (int32_t*)workspace;
  int32_t* slot_rank =
      (int32_t*)((unsigned char*)workspace + ws_tile_bytes(T, E));
  const int nt = num_tiles(T);
  if (stage == kRouteNeedPlan)
    return launch_plan(topk_idx, T, k, E, pad, counts, offsets, workspace, s);
  if (stage == kRouteNeedScan)
    return launch_scan(tile_base, nt, E, pad, counts, offsets, s);
  int32_t* gtot = ws_groups(workspace, T, E, k);
  if (stage == kRouteNeedGroupHist) {
    hipLaunchKernelGGL(tile_histogram_kernel, dim3(nt), dim3(256), 0, s,
                       topk_idx, T, k, E, tile_base, slot_rank, gtot);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
#define MOE_SCAN_G(PERV)                                                      \
  hipLaunchKernelGGL(expert_scan_groups_kernel<PERV>, dim3(num_groups(T)),    \
                     dim3(256), 0, s, tile_base, nt, E, pad, gtot,            \
                     num_groups(T), counts, offsets)
  if (E <= 256) MOE_SCAN_G(1);
  else if (E <= 512) MOE_SCAN_G(2);
  else MOE_SCAN_G(4);
#undef MOE_SCAN_G
  return hipGetLastError();
}

// The gate kernels of moe_route; *stage says what remains (plan or scan).
static hipError_t launch_gate(const void* x, const void* w, int xdt,
                              const float* bias, int T, int H, int E, int k,
                              int32_t* topk_idx, float* topk_w,
                              float* logits_dbg, void* workspace, int* stage,
                              hipStream_t s) {
  int32_t* tile_base = (int32_t*)workspace;
  int32_t* slot_rank =
      (int32_t*)((unsigned char*)workspace + ws_tile_bytes(T, E));
  *stage = kRouteNeedPlan;
  if (xdt == DT_BF16)
    return launch_gate_typed<uint16_t>(
        (const uint16_t*)x, (const uint16_t*)w, bias, T, H, E, k, topk_idx,
        topk_w, logits_dbg, tile_base, slot_rank, stage, s);
  return launch_gate_typed<float>((const float*)x, (const float*)w, bias, T,
                                  H, E, k, topk_idx, topk_w, logits_dbg,
                                  tile_base, slot_rank, stage, s);
}

hipError_t launch_route(const void* x, const void* w, int xdt,
                        const float* bias, int T, int H, int E, int k,
                        int pad, int32_t* topk_idx, float* topk_w,
                        int32_t* counts, int32_t* offsets, float* logits_dbg,
                        void* workspace, hipStream_t s) {
  if (T == 0)
    return launch_plan(topk_idx, T, k, E, pad, counts, offsets, workspace, s);
  int stage = kRouteNeedPlan;
  hipError_t err = launch_gate(x, w, xdt, bias, T, H, E, k, topk_idx, topk_w,
                               logits_dbg, workspace, &stage, s);
  if (err != hipSuccess) return err;
  return finish_plan(stage, topk_idx, T, k, E, pad, counts, offsets,
                     workspace, s);
}

// moe_route then moe_dispatch.  When the top-k leaves the plan to do for at
// most kSmallPlanT tokens, the plan kernel is skipped: the scatter launch
// rebuilds the plan in every workgroup (one launch fewer on the decode
// path); otherwise the two calls' launches as they are.
hipError_t launch_route_dispatch(const void* x, const void* w, int xdt,
                                 const float* bias, int T, int H, int E,
                                 int k, int pad, int32_t* topk_idx,
                                 float* topk_w, int32_t* counts,
                                 int32_t* offsets, float* logits_dbg,
                                 void* workspace, int pdt, void* rows,
                                 size_t capacity, float* row_scales,
                                 int32_t* row_src, int32_t* tok_row,
                                 hipStream_t s) {
  hipError_t err;
  if (T > 0 && T <= kSmallPlanT) {
    int stage = kRouteNeedPlan;
    err = launch_gate(x, w, xdt, bias, T, H, E, k, topk_idx, topk_w,
                      logits_dbg, workspace, &stage, s);
    if (err != hipSuccess) return err;
    // (its plan in LDS holds T / 64 x E bitmaps and first rows: up to 512
    // experts)
    if (stage == kRouteNeedPlan && E <= kGateWideE)
      return launch_plan_dispatch_small(x, xdt, T, H, topk_idx, k, E, pad,
                                        counts, offsets, pdt, rows, capacity,
                                        row_scales, row_src, tok_row, s);
    err = finish_plan(stage, topk_idx, T, k, E, pad, counts, offsets,
                      workspace, s);
  } else {
    err = launch_route(x, w, xdt, bias, T, H, E, k, pad, topk_idx, topk_w,
                       counts, offsets, logits_dbg, workspace, s);
  }
  if (err != hipSuccess) return err;
  if (T == 0 && capacity == 0) return hipSuccess;
  return launch_dispatch(x, xdt, T, H, topk_idx, k, E, counts, offsets,
                         workspace, pdt, rows, capacity, row_scales, row_src,
                         tok_row, s);
}

// The one-launch path's grid: at most one workgroup per compute unit (so all
// are resident together), a multiple of 8.  Its arrival count per GPU is
// kept on the host: the device counters start at 0 and grow by 2 G a call.
namespace {
constexpr int kOneLaunchMaxDevices = 64;
std::atomic<unsigned long long> g_one_launch_arrivals[kOneLaunchMaxDevices];
std::atomic<int> g_one_launch_cus[kOneLaunchMaxDevices];
}  // namespace

hipError_t launch_route_dispatch_one_launch(
    const void* x, const void* w, const float* bias, int T, int H, int E,
    int k, int pad, int32_t* topk_idx, float* topk_w, int32_t* counts,
    int32_t* offsets, float* logits_dbg, void* workspace, int pdt, void* rows,
    size_t capacity, float* row_scales, int32_t* row_src, int32_t* tok_row,
    hipStream_t s) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kOneLaunchMaxDevices) return hipErrorInvalidDevice;
  int cus = g_one_launch_cus[dev].load();
  if (cus == 0) {
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                                dev);
    if (err != hipSuccess) return err;
    g_one_launch_cus[dev].store(cus);
  }
  // the split gate's geometry for few tokens (as launch_gate_typed)
  const int epw = gate_epw(E);
  const int tiles = (T + 31) / 32;
  const int eg = epw;
  int S = (224 + tiles * eg - 1) / (tiles * eg);
  S = std::min(S, std::min(split_max(T), (H + 63) / 64));
  const int KR = ((H + S - 1) / S + 63) / 64 * 64;
  S = (H + KR - 1) / KR;
  const int ngate = tiles * S * eg;
  const int G = std::min((ngate + 7) / 8 * 8, cus / 8 * 8);
  if (G < 8) return hipErrorInvalidConfiguration;
  float* part = (float*)((unsigned char*)workspace + ws_tile_bytes(T, E) +
                         ws_rank_bytes(T, k));
  const ScatterShape g = scatter_shape(DT_BF16, pdt, T, H, false);
  const size_t lds = local_plan_lds_bytes(T, E);
  const unsigned long long gbase =
      g_one_launch_arrivals[dev].fetch_add(2ull * (unsigned long long)G);
  const uint16_t* xb = (const uint16_t*)x;
  const uint16_t* wb = (const uint16_t*)w;
  unsigned char* rb = (unsigned char*)rows;
  const long long cap = (long long)capacity;
#define MOE_OL(C4V, KV, MV)                                                    \
  hipLaunchKernelGGL((route_dispatch_one_launch_kernel<C4V, KV, MV>), dim3(G), \
                     dim3(256), lds, s, xb, wb, bias, T, H, E, k, pad, KR, S,  \
                     tiles, eg, part, topk_idx, topk_w, logits_dbg, counts,    \
                     offsets, rb, cap, row_scales, row_src, tok_row,           \
                     g.tblocks, g.hs, gbase)
#define MOE_OL_M(C4V, KV)                                                      \
  do {                                                                         \
    if (g.mode == 0) MOE_OL(C4V, KV, 0);                                       \
    else MOE_OL(C4V, KV, 1);                                                   \
  } while (0)
#define MOE_OL_K(C4V)                                                          \
  do {                                                                         \
    if (k <= 1) MOE_OL_M(C4V, 1);                                              \
    else if (k <= 2) MOE_OL_M(C4V, 2);                                         \
    else if (k <= 4) MOE_OL_M(C4V, 4);                                         \
    else if (k <= 8) MOE_OL_M(C4V, 8);                                         \
    else MOE_OL_M(C4V, 16);                                                    \
  } while (0)
  if (epw <= 4) MOE_OL_K(1);
  else MOE_OL_K(2);
#undef MOE_OL_K
#undef MOE_OL_M
#undef MOE_OL
  err = hipGetLastError();
  // a grid that never ran adds nothing to the device counters
  if (err != hipSuccess)
    g_one_launch_arrivals[dev].fetch_sub(2ull * (unsigned long long)G);
  return err;
}

hipError_t launch_plan(const int32_t* topk_idx, int T, int k, int E, int pad,
                       int32_t* counts, int32_t* offsets, void* workspace,
                       hipStream_t s) {
  const int nt = num_tiles(T);
  int32_t* tile_base = (int32_t*)workspace;
  int32_t* slot_rank =
      (int32_t*)((unsigned char*)workspace + ws_tile_bytes(T, E));
  if (nt > 0 && T <= kSmallPlanT) {
    hipLaunchKernelGGL(plan_small_kernel, dim3(1), dim3(512), 0, s, topk_idx,
                       T, k, E, pad, counts, offsets, tile_base, slot_rank);
    return hipGetLastError();
  }
  if (nt > 0) {
    hipLaunchKernelGGL(tile_histogram_kernel, dim3(nt), dim3(256), 0, s,
                       topk_idx, T, k, E, tile_base, slot_rank, nullptr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return launch_scan(tile_base, nt, E, pad, counts, offsets, s);
}

}  // namespace moe
