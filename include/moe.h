/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE route -> dispatch -> combine
 * library.  Plain pointers and sizes only; no C++ or framework types cross it.
 *
 * One MoE layer transform on one GPU's share of the tokens and experts:
 *
 *   moe_route            router gate GEMM, softmax top-k with renormalised
 *                        weights, per-expert histogram, padded exclusive scan
 *   moe_plan             the histogram and scan alone, for top-k choices made
 *                        elsewhere
 *   moe_dispatch         stable scatter of token rows into an expert-major
 *                        buffer padded per expert (optionally OCP fp8 E4M3
 *                        with one fp32 scale per 1x128 block)
 *   moe_route_dispatch   moe_route + moe_dispatch in one call (small decode
 *                        batches skip the plan kernel)
 *   moe_route_dispatch_one_launch
 *                        the same as one kernel launch (decode batches)
 *   moe_dispatch_noalloc moe_dispatch with no workspace argument (its scratch is
 *                        a static device array), for callers that cannot
 *                        allocate
 *   moe_combine_residual weighted gather-combine back to token order, fused
 *                        with the FarSkip-Collective dual residual update
 *   moe_farskip_aux      the auxiliary residual stream alone (split form)
 *   moe_combine_backward, moe_dispatch_backward
 *                        gradients through the same routing plan
 *   moe_expert_gemm_fp8  fp8 grouped GEMM of every expert over its segment
 *                        of the dispatched buffer (1x128 activation scales,
 *                        128x128 weight blocks)
 *   moe_expert_fixture   a stand-in expert (y = sigma_e * row) for tests and
 *                        benchmarks; not part of the transform
 *
 * Conventions shared by every entry point
 *   - Device pointers.  Every array argument is device memory (HBM) that the
 *     caller allocated and owns; the library never allocates, frees or keeps
 *     a pointer after the call returns.  Its only device memory of its own
 *     is the static scratch array of moe_dispatch_noalloc and the wait
 *     counters of moe_route_dispatch_one_launch.  Arrays are dense
 *     row-major with the shapes given below.  Arrays read or written as 16-byte vectors (x,
 *     w_gate, rows, y, shared, residuals, out, gradients of those, workspace)
 *     need 16-byte aligned base addresses; the others their element size.
 *   - Asynchrony.  Each call validates its arguments on the host, then only
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the null stream)
 *     and returns.  No call synchronises the device or copies device data to
 *     the host: the number of rows actually used stays on the device in
 *     offsets[E] (the pages' reason: host synchronisation and metadata
 *     broadcasts are what make stock all-to-all unsuitable; "Efficient and
 *     Portable Mixture-of-Experts Communication", section Sharding and
 *     Parallelism).
 *   - Errors.  A call returns MOE_OK or a negative moe_status.  Argument
 *     errors are detected before anything is enqueued and leave every output
 *     untouched; MOE_ERR_HIP reports a failed launch (see moe_last_hip_error).
 *     T == 0 is valid and enqueues nothing except what the entry point says.
 *   - Non-finite data.  The arithmetic is specified for finite inputs, and
 *     no call scans its data for NaN or infinities: they propagate (a NaN
 *     logit ranks above +Inf; an infinite element gives its fp8 block an
 *     infinite scale).  Whatever the data, every kernel keeps its accesses
 *     in bounds: expert ids outside [0, E) and rows outside the buffer are
 *     skipped, not followed.
 *   - Determinism.  No floating-point atomics are used: identical inputs give
 *     bit-identical outputs on every run.
 *   - Thread safety.  The library keeps no mutable state besides the last
 *     HIP error code (thread-local), for moe_dispatch_noalloc its static
 *     scratch array and that array's device address per GPU, and for
 *     moe_route_dispatch_one_launch its wait counters per GPU (device) and
 *     their running total (host, atomic).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  MOE_FP8_E4M3 is the OCP 8-bit E4M3 ("FN") format: bias 7,
 * max finite 448, subnormals down to 2^-9, NaN = S.1111.111, no infinities. */
typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8_E4M3 = 2
} moe_dtype;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,      /* a required pointer is NULL                     */
  MOE_ERR_SHAPE = -2,     /* a size is out of range or inconsistent         */
  MOE_ERR_DTYPE = -3,     /* an unsupported dtype or dtype combination      */
  MOE_ERR_ALIGN = -4,     /* a pointer is not 16-byte aligned               */
  MOE_ERR_CAPACITY = -5,  /* rows_capacity < moe_rows_capacity(T, E, k, pad) */
  MOE_ERR_WORKSPACE = -6, /* workspace_bytes < moe_workspace_bytes(T, E, k)  */
  MOE_ERR_ALIAS = -7,     /* an output overlaps an input it may not alias   */
  MOE_ERR_HIP = -8,       /* a kernel launch failed                         */
  MOE_ERR_SCRATCH = -9    /* sizes need more than the library's static
                             scratch (MOE_NOALLOC_SCRATCH_BYTES)            */
} moe_status;

/* Static description of a status code (never NULL). */
const char* moe_status_string(int status);

/* hipError_t of the last MOE_ERR_HIP returned on the calling thread. */
int moe_last_hip_error(void);

/* Largest number of experts and of experts per token the kernels accept. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 16

/*
 * Rows the expert-major buffer must provide: T*k + E*(pad-1).
 * Every (token, slot) pair gets its own row and each expert's segment is
 * rounded up to a multiple of `pad`, so this bound always suffices and
 * every writer gets a unique row without synchronising with any other --
 * the fixed upper bound per expert of "Efficient and Portable
 * Mixture-of-Experts Communication", section Portable Kernels, with the
 * per-expert padding `token_padding` of the "MoonEP developer guide" (core
 * configuration parameters).  Returns 0 for invalid sizes.
 */
size_t moe_rows_capacity(int T, int E, int k, int pad);

/* Bytes of scratch that moe_route / moe_plan write and moe_dispatch reads
 * (per-tile expert counts and prefixes, per-slot ranks, and for up to
 * 65536 tokens room for partial gate logits when the gate splits the hidden
 * dimension).  A workspace belongs to one route -> dispatch sequence at
 * a time: calls in flight on different streams need different workspaces.
 * 0 if T == 0. */
size_t moe_workspace_bytes(int T, int E, int k);

/*
 * moe_route -- router gate, softmax top-k, per-expert histogram and scan.
 *
 * The router is a small linear layer producing a probability distribution
 * over the experts; the top-k experts are selected and later weighted by
 * that distribution ("Efficient and Portable Mixture-of-Experts
 * Communication", Introduction).  Counting the tokens bound for each expert
 * follows the same page's section Dispatch; the padded exclusive scan gives
 * MoonEP's `cu_seqlens` with `token_padding` ("MoonEP developer guide", core
 * API example and core configuration parameters).
 *
 *   x        [T, H] x_dtype (MOE_F32 or MOE_BF16), token activations
 *   w_gate   [E, H] x_dtype, router weight (row e = expert e)
 *   bias     [E] fp32 added to the logits before the softmax, or NULL
 *   k        experts per token, 1 <= k <= min(E, MOE_MAX_TOPK)
 *   pad      per-expert row padding (>= 1)
 * outputs
 *   topk_idx [T, k] int32  chosen experts, by descending logit; equal logits
 *                          rank the lower expert index first
 *   topk_w   [T, k] fp32   softmax weights renormalised over the k chosen
 *                          (= softmax over the k chosen logits)
 *   counts   [E] int32     (token, slot) pairs routed to each expert
 *   offsets  [E+1] int32   offsets[0] = 0, offsets[e+1] = offsets[e] +
 *                          ceil(counts[e]/pad)*pad; offsets[E] = rows used
 *   logits_dbg [T, E] fp32 or NULL: the logits (bias included) that the
 *                          selection ranked, for stage-wise checking
 *   workspace  device scratch of workspace_bytes >= moe_workspace_bytes(T,E,k);
 *              read by the next moe_dispatch of the same tokens
 * Logits are accumulated in fp32 on the matrix cores (bf16 or fp32 inputs).
 * Limits: 1 <= E <= MOE_MAX_EXPERTS, H % 8 == 0, H >= 8; above 512 experts
 * x must be bf16 (MOE_ERR_DTYPE) and T <= 65536 (MOE_ERR_SHAPE).
 */
int moe_route(const void* x, int x_dtype, int T, int H,
              const void* w_gate, int E, const float* bias,
              int k, int pad,
              int32_t* topk_idx, float* topk_w,
              int32_t* counts, int32_t* offsets,
              float* logits_dbg,
              void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * moe_plan -- histogram and padded scan for top-k choices made elsewhere
 * (MoonEP's dispatch takes the chosen experts as input: "MoonEP developer
 * guide", core API example).  Same outputs and workspace contract as the
 * histogram/scan part of moe_route.
 *   topk_idx [T, k] int32, each entry in [0, E) and distinct within a row;
 *            an entry outside [0, E) is counted for no expert and its slot
 *            later receives no row.
 */
int moe_plan(const int32_t* topk_idx, int T, int k, int E, int pad,
             int32_t* counts, int32_t* offsets,
             void* workspace, size_t workspace_bytes,
             void* stream);

/*
 * moe_dispatch -- stable scatter of token rows into the expert-major buffer.
 *
 * Tokens are copied into contiguous per-expert buffers that feed the
 * experts, and the row each (token, slot) copy went to is kept for the
 * combine ("Efficient and Portable Mixture-of-Experts Communication",
 * sections Dispatch and Combine).  Unlike that design's atomically
 * incremented receive counter, the order is fixed: expert e's segment
 * [offsets[e], offsets[e] + counts[e]) holds its tokens in ascending token
 * order.  fp8 payloads carry block scaling factors (same page, Dispatch;
 * FP8 dispatch in the DeepEP announcement, technical overview).
 *
 *   x, x_dtype, T, H      as for moe_route
 *   topk_idx, k, E, pad   as produced by moe_route / moe_plan
 *   counts, offsets       from the same moe_route / moe_plan call
 *   workspace             from the same moe_route / moe_plan call
 *   payload_dtype         x_dtype (exact copy), or MOE_FP8_E4M3 for bf16 or
 *                         fp32 x (requires H % 128 == 0)
 * outputs
 *   rows       [rows_capacity, H] payload_dtype; rows holding no token are
 *              not written
 *   row_scales [rows_capacity, H/128] fp32 for fp8 payloads (else NULL): for
 *              each 128-wide block b of a row, s = fl32(amax / 448) (1 if the
 *              block is all zero) and row = E4M3(fl32(x / s)), round to
 *              nearest even, saturating
 *   row_src    [rows_capacity] int32: token held by each row, -1 for padding
 *              rows and for every row at or beyond offsets[E]
 *   tok_row    [T, k] int32: row that received slot (t, j)
 * rows_capacity must be >= moe_rows_capacity(T, E, k, pad).
 */
int moe_dispatch(const void* x, int x_dtype, int T, int H,
                 const int32_t* topk_idx, int k, int E, int pad,
                 const int32_t* counts, const int32_t* offsets,
                 const void* workspace, size_t workspace_bytes,
                 int payload_dtype,
                 void* rows, size_t rows_capacity, float* row_scales,
                 int32_t* row_src, int32_t* tok_row,
                 void* stream);

/*
 * moe_route_dispatch -- moe_route followed by moe_dispatch in one call, for
 * the low-latency path of small decode batches (DeepEP's low-latency kernels
 * for small decode batches: DeepEP release news, technical overview).  The
 * arguments are the union of the two calls' (same meaning, layout and
 * limits); the outputs are bit-identical to moe_route then moe_dispatch on
 * the same stream.  Up to 512 tokens the plan kernel between top-k and
 * scatter is skipped: every scatter workgroup rebuilds the plan (tile
 * ballots, counts, padded scan) in its own LDS from topk_idx, so route +
 * scatter take one launch fewer (moe_route_dispatch_one_launch, below,
 * replaces the remaining boundaries by grid-wide waits and measured slower
 * on MI355X).
 * The workspace is then scratch of this call only: it does not hold a plan
 * a later moe_dispatch could read.  Errors as for the two calls.
 */
int moe_route_dispatch(const void* x, int x_dtype, int T, int H,
                       const void* w_gate, int E, const float* bias,
                       int k, int pad,
                       int32_t* topk_idx, float* topk_w,
                       int32_t* counts, int32_t* offsets,
                       float* logits_dbg,
                       void* workspace, size_t workspace_bytes,
                       int payload_dtype,
                       void* rows, size_t rows_capacity, float* row_scales,
                       int32_t* row_src, int32_t* tok_row,
                       void* stream);

/*
 * moe_route_dispatch_one_launch -- moe_route_dispatch as one kernel launch,
 * the form of DeepEP's low-latency path for small decode batches (DeepEP
 * release news, technical overview): gate partial sums, top-k and the
 * scatter run in one grid whose workgroups wait for each other twice (after
 * the partial sums, after the top-k) at device-scope counters.  Same
 * arguments, outputs and errors as moe_route_dispatch, and additionally
 * x_dtype must be MOE_BF16 (else MOE_ERR_DTYPE), T <= 256 and E <= 512
 * (else MOE_ERR_SHAPE).  The results equal moe_route_dispatch's up to the
 * rounding order of the partial-sum reduction (4 waves per token instead of
 * 8): the logits may differ in the last bits, so choices at exact near-ties
 * may differ; rows, ranks and weights follow the top-k it made.
 * Requirements: `stream` belongs to the calling thread's current device
 * (the device whose counters the call uses); the grid holds at most one
 * workgroup per compute unit, so all are resident; calls of this entry
 * point must not overlap on one GPU
 * (the wait counters are per GPU and only grow; overlapping calls could
 * give wrong results, never a hang: each wait is bounded).  On MI355X it
 * measured slower than moe_route_dispatch, which stays the decode path.
 */
int moe_route_dispatch_one_launch(const void* x, int x_dtype, int T, int H,
                                  const void* w_gate, int E,
                                  const float* bias, int k, int pad,
                                  int32_t* topk_idx, float* topk_w,
                                  int32_t* counts, int32_t* offsets,
                                  float* logits_dbg,
                                  void* workspace, size_t workspace_bytes,
                                  int payload_dtype,
                                  void* rows, size_t rows_capacity,
                                  float* row_scales,
                                  int32_t* row_src, int32_t* tok_row,
                                  void* stream);

/*
 * moe_dispatch_noalloc -- moe_dispatch for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc) and have no workspace to hand over: same arguments and outputs
 * as moe_dispatch without workspace / workspace_bytes, bit-identical rows,
 * row_scales, row_src and tok_row.  The tile plan moe_dispatch reads from the
 * workspace (per-(tile, expert) first rows, per-slot ranks) is rebuilt from
 * topk_idx in a static device array of MOE_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends; nothing is
 * allocated or freed.  That array is shared by every call on the same GPU:
 * calls that overlap on one GPU (other streams, other host threads) race on
 * it and must be serialised by the caller.  Its contents do not carry over
 * between calls (each call rewrites what it reads).
 * Limit: moe_noalloc_scratch_bytes(T, E, k) <= MOE_NOALLOC_SCRATCH_BYTES
 * (8 MiB: about 4 bytes per slot plus 4 bytes per expert per 64 tokens;
 * 65536 tokens fit for every E <= 512 with k <= 16 and E <= 1024 with
 * k <= 8), else MOE_ERR_SCRATCH
 * before anything is enqueued.  Other errors as for moe_dispatch; MOE_ERR_HIP also
 * if the array's device address cannot be obtained.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
size_t moe_noalloc_scratch_bytes(int T, int E, int k);
int moe_dispatch_noalloc(const void* x, int x_dtype, int T, int H,
                         const int32_t* topk_idx, int k, int E, int pad,
                         const int32_t* counts, const int32_t* offsets,
                         int payload_dtype,
                         void* rows, size_t rows_capacity, float* row_scales,
                         int32_t* row_src, int32_t* tok_row,
                         void* stream);

/*
 * moe_combine_residual -- weighted gather-combine fused with the FarSkip
 * dual residual update.
 *
 * routed[t] = sum_{j<k} topk_w[t,j] * y[tok_row[t,j]], accumulated in fp32
 * with j ascending: the weighted average of the selected experts' outputs,
 * with the accumulation fused into the gather ("Efficient and Portable
 * Mixture-of-Experts Communication", Introduction, Sharding and Parallelism,
 * Combine).  With a residual, the update of the Instella-MoE article (where
 * the dual residual streams are implemented): the MoE output is routed +
 * shared, residual_no_routed = residual + shared, residual = residual + MoE
 * output; each output is rounded once from fp32 to bf16 (nearest even).
 *
 *   y         [y_rows, H] y_dtype (MOE_BF16 or MOE_F32): expert outputs in the
 *             dispatch row order; a slot whose tok_row lies outside
 *             [0, y_rows) contributes nothing
 *   tok_row   [T, k] int32 from moe_dispatch;  topk_w [T, k] fp32
 *   shared    [T, H] bf16 shared-expert output, or NULL (= 0)
 * dual-residual form (residual_in != NULL):
 *   residual_in        [T, H] bf16
 *   residual_out       [T, H] bf16 = bf16(residual + routed + shared); may be
 *                      the same pointer as residual_in (in-place update)
 *   residual_no_routed [T, H] bf16 = bf16(residual + shared), or NULL when
 *                      moe_farskip_aux produced it earlier (split form: the
 *                      auxiliary stream does not wait for the routed combine)
 *   out must be NULL
 * routed-only form (residual_in == NULL):
 *   out [T, H] out_dtype (MOE_BF16 or MOE_F32) = routed + shared
 *   residual_out and residual_no_routed must be NULL
 */
int moe_combine_residual(const void* y, int y_dtype, int H, size_t y_rows,
                         const int32_t* tok_row, const float* topk_w,
                         int T, int k,
                         const void* shared,
                         const void* residual_in,
                         void* residual_out,
                         void* residual_no_routed,
                         void* out, int out_dtype,
                         void* stream);

/*
 * moe_farskip_aux -- the auxiliary residual stream alone:
 *   residual_no_routed[T, H] = bf16(residual_in + shared)   (shared NULL = 0)
 * The FarSkip-Collective dual residual streams (Instella-MoE article, the
 * dual residual streams and the four-line update) let the next layer's
 * attention read this stream while the routed combine is still pending, so
 * it can be produced before routing; the main stream then comes from
 * moe_combine_residual with residual_no_routed = NULL.  Bit-identical to the
 * fused form.  All arrays bf16 [T, H]; the output may not overlap the inputs.
 */
int moe_farskip_aux(const void* shared, const void* residual_in,
                    void* residual_no_routed, int T, int H, void* stream);

/*
 * moe_combine_backward -- gradient of the weighted combine through the
 * routing plan of the forward pass (MoonEP's backward reuses the forward
 * plan: "MoonEP developer guide", core API example, backward).
 * With routed[t] = sum_j topk_w[t,j] * y[tok_row[t,j]] and an upstream
 * gradient grad_out = dL/d routed ([T, H] bf16; for the dual residual form
 * this is the gradient of residual_out):
 *   grad_y[tok_row[t,j]] = bf16(topk_w[t,j] * grad_out[t])   [y_rows, H] bf16
 *   grad_w[t,j] = sum_h grad_out[t,h] * y[tok_row[t,j],h]   [T, k] fp32
 * Rows of grad_y that no slot references are not written.  y_dtype is
 * MOE_BF16 or MOE_F32.  Sums are fp32 in a fixed order (deterministic).
 */
int moe_combine_backward(const void* grad_out, const void* y, int y_dtype,
                         int H, size_t y_rows, const int32_t* tok_row,
                         const float* topk_w, int T, int k, void* grad_y,
                         float* grad_w, void* stream);

/*
 * moe_dispatch_backward -- gradient of the scatter: every row is a copy of
 * its token, so grad_x[t] = sum_j grad_rows[tok_row[t,j]] (an unweighted
 * combine; slots whose row lies outside [0, rows_capacity) add nothing).
 *   grad_rows [rows_capacity, H] rows_dtype (MOE_BF16 or MOE_F32)
 *   grad_x    [T, H] grad_x_dtype (MOE_BF16 or MOE_F32), fp32 accumulation
 */
int moe_dispatch_backward(const void* grad_rows, int rows_dtype, int H,
                          size_t rows_capacity, const int32_t* tok_row, int T,
                          int k, void* grad_x, int grad_x_dtype,
                          void* stream);

/*
 * moe_expert_gemm_fp8 -- grouped GEMM of every expert over its segment of
 * the fp8 expert-major buffer, in the form dispatch writes it (the grouped
 * GEMM between dispatch and combine: "Efficient and Portable
 * Mixture-of-Experts Communication", Dispatch; FP8 tokens with block scaling
 * factors: DeepEP news, technical overview).  For every row r of expert e's
 * segment [offsets[e], offsets[e+1]) and every n < N:
 *   y[r, n] = sum_b row_scales[r, b] * w_scales[e, n/128, b]
 *             * sum_{h = 128b}^{128b+127} E4M3(rows[r, h]) * E4M3(w[e, n, h])
 * in fp32 (each 128-wide block's fp8 products summed by the matrix core, then
 * scaled and added in block order), stored as fp32 or rounded once to bf16.
 *   rows       [rows_capacity, K] OCP E4M3 codes; row_scales [rows_capacity,
 *              K/128] fp32 (moe_dispatch's fp8 output)
 *   row_src    [rows_capacity] int32 or NULL: rows with row_src < 0 (padding)
 *              are stored as zeros
 *   offsets    [E+1] int32 from moe_route / moe_plan (device)
 *   w          [E, N, K] E4M3 codes; w_scales [E, N/128, K/128] fp32
 *   y          [rows_capacity, N] y_dtype (MOE_BF16 or MOE_F32); rows outside
 *              every segment are not written
 *   workspace  >= moe_expert_gemm_workspace_bytes(rows_capacity, E) bytes
 * K and N multiples of 128, K <= 8192, rows_capacity * K and N * K below
 * 2^32 (MOE_ERR_SHAPE otherwise).  Segment bounds are clamped to
 * rows_capacity.
 */
size_t moe_expert_gemm_workspace_bytes(size_t rows_capacity, int E);
int moe_expert_gemm_fp8(const void* rows, const float* row_scales, int K,
                        size_t rows_capacity, const int32_t* row_src,
                        const int32_t* offsets, int E, const void* w,
                        const float* w_scales, int N, void* y, int y_dtype,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * moe_expert_fixture -- stand-in expert used by tests and benchmarks in
 * place of the grouped expert GEMM that sits between dispatch and combine
 * ("Efficient and Portable Mixture-of-Experts Communication", Dispatch: the
 * per-expert buffers feed a grouped GEMM).  Not part of the transform.
 *   y[r] = sigma[e] * deq(rows[r]) for every row r < rows_capacity with
 *   row_src[r] >= 0, where e is the expert whose segment
 *   [offsets[e], offsets[e+1]) holds r and deq(q) = q * row_scales[r, b] for
 *   fp8 (an fp32 product), the stored value otherwise; y is stored as fp32
 *   or rounded once to bf16.  Rows with row_src[r] < 0 are set to zero.
 */
int moe_expert_fixture(const void* rows, int payload_dtype,
                       const float* row_scales, int H,
                       const int32_t* row_src, const int32_t* offsets, int E,
                       const float* sigma, size_t rows_capacity,
                       void* y, int y_dtype,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
