/*
 * moelora.h -- C ABI of the routed MoE expert layer with rank-r side-LoRA
 * (forward and backward) on one AMD MI355X (gfx950).
 *
 * What the calls compute follows DeepGEMM PR #9 "feat(mega): add fused shared
 * side-LoRA kernels" (section "Historical implementation": Summary and
 * Correctness coverage) and PR #17 "Align MegaMoE training with upgraded
 * K-grouped TMA and layouts" (Summary):
 *   - routes are dispatched into an expert-contiguous pool, each expert padded
 *     to BLOCK_M rows, padding rows zeroed;
 *   - per route (t, j) with expert e and u = x_t:
 *       g = W1_e u + s B1_e (A1 u),  v = W3_e u + s B3_e (A3 u),
 *       h = silu(g) * v,             y = W2_e h + s B2 (A2_e h),
 *       out_t = sum_j w[t, j] y_(t, j)
 *     with A1, A3, B2 shared by all experts and B1, B3, A2 expert-local;
 *   - the backward returns grad-x and the router gradients in source-token
 *     order and the six adapter gradients (no frozen-weight gradients unless
 *     asked for), with padding rows kept out of every reduction;
 *   - unsupported modes and short workspaces are rejected before any launch.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers, row-major, densely packed, and
 *     16-byte aligned.  bf16 is stored as uint16 bit patterns.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     keeps a pointer after a call returns.
 *   - Work is queued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting for the device.
 *   - Arguments are validated on the host first.  On any error nothing is
 *     written and no kernel is launched.
 *   - Outputs are overwritten, never accumulated; empty experts and dropped
 *     routes get exact zeros.
 *   - Calls that share a workspace or outputs must be ordered on one stream.
 *   - The forward and backward run independent parts of their work on a
 *     second stream of the device that the library creates on first use
 *     (non-blocking, default priority), ordered against the caller's stream
 *     by events: it waits for the caller's stream at the call's start, and
 *     the caller's stream waits for it before the call's last kernel, so in
 *     the caller's stream order the call's work is complete as before.
 *     Calls on one device hold a host lock while they enqueue.  While the
 *     caller's stream is being captured into a graph, and in
 *     moe_lora_forward_noalloc, every kernel runs on the caller's stream.
 */
#ifndef MOELORA_H
#define MOELORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_ERR_INVALID (-1)     /* bad shape, pointer, alignment or pool */
#define MOE_ERR_UNSUPPORTED (-2) /* a mode this build does not implement */
#define MOE_ERR_WORKSPACE (-3)   /* saved/scratch buffer smaller than required */
#define MOE_ERR_HIP (-4)         /* a HIP launch or attribute call failed */

#define MOE_ACT_SWIGLU 0         /* h = silu(g) * v, silu(g) = g sigmoid(g) */
#define MOE_ACT_GEGLU 1          /* h = gelu(g) * v, gelu(g) = g Phi(g) (exact GELU,
                                    Phi the standard normal distribution function);
                                    other values: UNSUPPORTED */
#define MOE_BASE_BF16 0          /* W13 / W2 in bf16 */
#define MOE_BASE_MXFP4 1         /* W13 / W2 as e2m1 with e8m0 scales per 32 along K */

/* Device status word of the saved workspace: the int32 at byte offset
 * MOE_SAVED_STATUS_OFFSET of `saved`, cleared by every moe_lora_forward and
 * raised by its kernels (read it after the forward, on the same stream).
 *   MOE_SAVED_FP16_RANGE  the gate/up pre-activations g, v are saved in fp16
 *     for the backward.  Without a clamp they must stay below 65504 in
 *     magnitude; the bit is set when some |g| or |v| reached 65520 or more
 *     (it rounds to infinity in fp16).  The forward's `out` is still right
 *     (the activation uses the fp32 values) but a backward from this saved
 *     state returns non-finite gradients.  With a clamp 0 < c < 65504 such
 *     values are clipped to c like any other value beyond it, and the bit is
 *     never set. */
#define MOE_SAVED_STATUS_OFFSET 0
#define MOE_SAVED_FP16_RANGE 1

/* Shape and options of one layer call.
 *   T tokens, H hidden, I intermediate, E local experts, topk routes per token,
 *   rank r of the side adapters, scale s of the adapter deltas (0 => plain MoE).
 *   block_m: pool padding granularity; 0 asks the library (see moe_lora_block_m),
 *     otherwise one of 16, 32, 64, 96, 128, 192, 240.
 *   activation: MOE_ACT_SWIGLU or MOE_ACT_GEGLU (the gated activations the
 *     pages list: PR #17 Summary; PR #9, "Correctness coverage").
 *   clamp: activation clamp c: when 0 < c < +inf both pre-activations are
     clipped to [-c, c] before the gated activation, h = f(clip(g)) clip(v),
     and the clip passes the gradient only where |x| <= c (the pages name the
     clamp -- PR #9 "Correctness coverage", production clamp = 10 -- without
     defining it; this is the plainest reading).  c <= 0 or +inf: no clamp;
     NaN: MOE_ERR_INVALID.  The clip decision is taken on the fp16-rounded
     pre-activation the forward saves, so forward and backward agree.
 * Supported: T >= 1, H % 256 == 0, I % 256 == 0, 1 <= E <= 512,
 *   1 <= topk <= 16, 1 <= rank <= 256 (a rank that is not a multiple of 8
 *   runs on copies of the factors widened with zero rows or columns to the
 *   next multiple, kept in the scratch workspace; the extra terms are exact
 *   zeros and the gradients are cut back to the caller's rank), T*H*2 and 4*I*H
 *   below 2^31 bytes (one 32-bit buffer offset per token-row tensor and per
 *   expert's weights).  Other values: MOE_ERR_UNSUPPORTED (non-positive sizes:
 *   MOE_ERR_INVALID).  base_format: MOE_BASE_BF16 or MOE_BASE_MXFP4. */
typedef struct moe_lora_desc {
  int32_t T, H, I, E, topk, rank;
  int32_t block_m;
  float scale;
  int32_t activation;
  float clamp;
  int32_t base_format;
} moe_lora_desc;

/* The dispatch pool written by build_pool (device int32 arrays).
 *   counts[E]          routes per expert
 *   offsets[E+1]       first pool row of each expert; offsets[E] = pool rows in use
 *   route_to_row[T*k]  pool row of route f = t*k + j, -1 if dropped
 *   row_to_route[capacity]  route of each pool row, -1 for padding and unused rows
 *   capacity           rows of row_to_route; must equal moe_lora_pool_capacity()
 *   block_m            the resolved BLOCK_M the pool was built with */
typedef struct moe_pool {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* route_to_row;
  const int32_t* row_to_route;
  int64_t capacity;
  int32_t block_m;
} moe_pool;

/* Layer parameters (device, bf16 unless noted; nn.Linear [out, in] layout):
 *   W13 [E, 2I, H]  rows 0..I-1 = W1 (gate), rows I..2I-1 = W3 (up)
 *   W2  [E, H, I]
 *   A1, A3 [r, H]   shared;   B1, B3 [E, I, r] expert-local
 *   A2  [E, r, I]   expert-local;   B2 [H, r] shared
 *   W13_scale, W2_scale: e8m0 block scales for MOE_BASE_MXFP4, NULL for bf16.
 *   W13T, W2T, W13P, W2P: optional transformed copies of the frozen base,
 *     written once by moe_lora_transform_base and reused by every call
 *     (PR #9 Summary: reusable transformed weights), in a layout private to
 *     the library: the weight tiles of one GEMM pipeline stage stored as the
 *     bytes it loads, one stage after another, so that each stage reads one
 *     contiguous block (32 KB of bf16, or 9 KB of MXFP4 codes and scales)
 *     instead of a short run from each of 256 rows.
 *       W13T, W2T: W13[e]^T, W2[e]^T for the backward's two data-gradient
 *         GEMMs, E x 2I x H and E x H x I bf16 values (for an MXFP4 base, of
 *         the dequantised values); without them (NULL) the backward
 *         transposes W13 / W2 on the fly (an MXFP4 base also expanded to
 *         bf16).  The forward ignores them.
 *       W13P, W2P: W13, W2 for the forward's two base GEMMs: E x 2I x H and
 *         E x H x I bf16 values; for MOE_BASE_MXFP4, E*2I*H*9/16 and
 *         E*H*I*9/16 bytes (the e2m1 codes and e8m0 scales).  The backward
 *         ignores them.
 *     Results are bitwise the same with or without any of them; their
 *     contents must come from moe_lora_transform_base on the same W13 / W2.
 *     Each may be given alone; 16-byte aligned. */
typedef struct moe_lora_params {
  const void* W13;
  const void* W2;
  const uint8_t* W13_scale;
  const uint8_t* W2_scale;
  const void *A1, *A3, *B1, *B3, *A2, *B2;
  const void* W13T;
  const void* W2T;
  const void* W13P;
  const void* W2P;
} moe_lora_params;

/* Gradient outputs (device bf16, same layouts as the parameters).  The six
 * adapter gradients are required.  dW13 [E, 2I, H] and dW2 [E, H, I] are the
 * optional frozen-weight gradients of the ordinary path (PR #9, "Matched
 * old/new performance"): dW13_e = sum over e's routes of [dg; dv] x_t^T,
 * dW2_e = sum of (w go_t) h^T, contracted over the expert's rows in pool
 * order; an expert without routes gets exact zeros.  NULL skips each; a
 * non-NULL pointer must be 16-byte aligned (else MOE_ERR_INVALID).  With an
 * MXFP4 base they are the gradients with respect to the dequantised
 * weights. */
typedef struct moe_lora_grads {
  void *dA1, *dA3, *dB1, *dB3, *dA2, *dB2;
  void *dW13, *dW2;
} moe_lora_grads;

/* Human-readable name of a status code (static string). */
const char* moe_lora_status_string(moe_status status);

/* Library version, e.g. 100 for 0.1.0. */
int32_t moe_lora_version(void);

/* BLOCK_M used for `desc` (resolves block_m == 0 to the library's choice).
 * PR #17 Summary: the block size is queried from the library, not duplicated
 * by callers; forward and backward use the same pool. */
moe_status moe_lora_block_m(const moe_lora_desc* desc, int32_t* block_m);

/* Rows of row_to_route to allocate: T*k + min(E, T*k) * (BLOCK_M - 1), the
 * largest pool any routing can produce. */
moe_status moe_lora_pool_capacity(const moe_lora_desc* desc, int64_t* rows);

/* Bytes of the two workspaces:
 *   saved   -- written by moe_lora_forward, read by moe_lora_backward; holds
 *              the status word (MOE_SAVED_STATUS_OFFSET), a copy of the layer
 *              input (the saved-X reuse of PR #9, "2026-09-20" -> What
 *              changed), the gate/up pre-activations in fp16 (|g|, |v| must
 *              stay below 65504 without a clamp: MOE_SAVED_FP16_RANGE) and
 *              the activations.
 *   scratch -- temporary space of moe_lora_forward and moe_lora_backward
 *              (nothing in it survives a call; both need the full size). */
moe_status moe_lora_workspace_size(const moe_lora_desc* desc, size_t* saved_bytes,
                                   size_t* scratch_bytes);

/* Build the dispatch pool from top-k expert ids (PR #9, "2026-09-21: restore
 * wide-K wgrad safely" -> Implementation: true physical expert offsets, groups
 * never rounded into a neighbour; "Historical implementation" -> Summary:
 * padding zeroed).
 *   topk_idx [T, k] int32: expert id, or -1 for a dropped route.  Ids outside
 *     [-1, E) are dropped as well and counted into *device_error (device
 *     int32, may be NULL), which the call overwrites.
 *   Rows of one expert follow ascending route index t*k + j (deterministic).
 *   counts, offsets, route_to_row, row_to_route: outputs as in moe_pool. */
moe_status build_pool(const moe_lora_desc* desc, const int32_t* topk_idx, int32_t* counts,
                      int32_t* offsets, int32_t* route_to_row, int32_t* row_to_route,
                      int64_t capacity, int32_t* device_error, void* stream);

/* Write the transformed base weights of moe_lora_params from params->W13 /
 * params->W2 (the adapter factors are not read): W13T and W2T (E*2I*H and
 * E*H*I bf16 values: the transposed weights for the backward; for
 * MOE_BASE_MXFP4 the dequantised weights e2m1 x 2^(e-127), exact in bf16,
 * read from the packed W13 / W2 and their scales, both required) and W13P,
 * W2P (the forward's weights: the same sizes for a bf16 base; for
 * MOE_BASE_MXFP4 E*2I*H*9/16 and E*H*I*9/16 bytes of codes and scales).
 * Any output may be NULL (skipped); outputs are 16-byte aligned device
 * buffers that overlap no input and no other output.  Queued on `stream`
 * like every call. */
moe_status moe_lora_transform_base(const moe_lora_desc* desc, const moe_lora_params* params, void* W13T,
                                   void* W2T, void* W13P, void* W2P, void* stream);

/* Two-term FP6 (E2M3) split of bf16 rows, the activation operand of the
 * MXFP4 base's scaled fp6 x fp4 matrix products (PR #9 "Historical
 * implementation" -> Summary: native MXFP4 base with bf16 side adapters, the
 * activations keeping bf16 precision).  moe_lora_forward runs it internally
 * on x and on the activations h; this call exposes it alone.
 *   src [rows, K] bf16 (K % 64 == 0, else MOE_ERR_UNSUPPORTED).
 *   Per row and aligned 32-block: s1 = 2^E1 with E1 the smallest integer such
 *   that max|x| <= 7.5 s1 (E1 = -127 for an all-zero block), q1 = E2M3(x/s1)
 *   rounded to nearest, ties to even (OCP MX v1.0 FP6 E2M3: bias 1,
 *   subnormals m/8, largest 7.5; code 8e + m, sign in bit 5), r = x - s1 q1
 *   (exact), (s2, q2) from r the same way; |x - (s1 q1 + s2 q2)| <=
 *   2^-8 max(|x|, s1).
 *   codes [rows, 2K bytes]: per 64-element chunk c, 128 bytes; term t (q1,
 *     then q2) at 64t; the 32 six-bit codes of the chunk's 32-block h packed
 *     into six little-endian dwords (element i in bits 6i .. 6i+5), dwords
 *     0-3 at 64t + 16h and dwords 4-5 at 64t + 32 + 8h; bytes 64t + 48 ..
 *     64t + 63 are not written;
 *   scale_words [K/64, rows] uint32 (stage-major: the words of one chunk
 *     for all rows are consecutive): per chunk, bytes {E1+127 of its first
 *     32-block, of its second, E2+127 of the first, of the second}.
 *   src, codes 16-byte aligned, scale_words 4-byte aligned, no overlaps. */
moe_status moe_lora_split_e2m3x2(const void* src, int64_t rows, int32_t K, void* codes, void* scale_words,
                                 void* stream);

/* Forward of the layer.
 *   x [T, H] bf16, topk_w [T, k] fp32 router weights (used as given),
 *   out [T, H] bf16 (overwritten), saved / scratch per moe_lora_workspace_size
 *   (16-byte aligned; a short one returns MOE_ERR_WORKSPACE).
 *   `pool` must come from build_pool with the same desc and topk ids.
 *   x, out and the workspaces must not overlap. */
moe_status moe_lora_forward(const moe_lora_desc* desc, const moe_pool* pool, const void* x,
                            const float* topk_w, const moe_lora_params* params, void* out,
                            void* saved, size_t saved_bytes, void* scratch, size_t scratch_bytes,
                            void* stream);

/* moe_lora_forward without a scratch argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, checks and results as
 * moe_lora_forward (bitwise); the forward's temporary tensors live instead in
 * a device array inside the library, 64 MiB on every device the library runs
 * on, held until the process ends.  The call allocates and frees nothing.
 *   - A layer whose forward needs more than 64 MiB of scratch returns
 *     MOE_ERR_WORKSPACE before any launch (the production share needs far
 *     more: use moe_lora_forward there; the token-sweep shapes up to a few
 *     hundred tokens fit).
 *   - All calls on one device share that device's array: calls that overlap
 *     on one device (different streams, concurrent threads) race.  Order them
 *     on one stream.
 *   - The first call on a device looks the array's address up (a HIP
 *     symbol query, no allocation); failure returns MOE_ERR_HIP. */
moe_status moe_lora_forward_noalloc(const moe_lora_desc* desc, const moe_pool* pool, const void* x,
                                    const float* topk_w, const moe_lora_params* params, void* out,
                                    void* saved, size_t saved_bytes, void* stream);

/* Backward of the layer for L = <grad_out, out>.
 *   grad_out [T, H] bf16; topk_w and params as given to the forward; `saved`
 *   as the forward left it (read only, may be reused by repeated calls).
 *   grad_x [T, H] bf16, grad_topk_w [T, k] fp32 (0 for dropped routes) and the
 *   gradients in `grads` are overwritten.  The result is a deterministic
 *   function of the inputs (bitwise repeatable). */
moe_status moe_lora_backward(const moe_lora_desc* desc, const moe_pool* pool,
                             const void* grad_out, const float* topk_w,
                             const moe_lora_params* params, const void* saved,
                             size_t saved_bytes, void* grad_x, float* grad_topk_w,
                             const moe_lora_grads* grads, void* scratch, size_t scratch_bytes,
                             void* stream);

/* ------------------------------------------------------------------------
 * Several adapters in one pass (OpenPipe/ART PR #1139, Behavior: several
 * adapters share one MoE pass; the router runs once per adapter; the
 * dispatched expert rows carry adapter IDs so that each adapter's own LoRA
 * factors serve its rows; Validation: the fused pass equals running the
 * adapters one after another, bit for bit).
 *
 * The T tokens of a call form `count` roots, one per adapter: root a is the
 * tokens offsets[a] .. offsets[a+1]-1 (contiguous; an empty root is
 * allowed), and every route of a token carries its root's adapter.  For each
 * root the calls compute exactly what the single-adapter calls above compute
 * on that root's tokens with adapter a's factors: outputs, grad-x and router
 * gradients by token, and each adapter's factor gradients over its own root
 * (an adapter with an empty root gets exact zeros).  The base W13 / W2 (and
 * W13T / W2T, the MXFP4 scales, s and every desc field) are common.
 *
 * Parameters and gradients are the single-adapter tensors stacked over the
 * adapters: A1, A3 [count, r, H]; B1, B3 [count, E, I, r]; A2 [count, E, r,
 * I]; B2 [count, H, r]; likewise dA1 .. dB2.  The frozen-weight gradients
 * dW13 / dW2 are not offered with count > 1 (MOE_ERR_UNSUPPORTED).
 *
 * The pool groups rows by (expert e, adapter a) as group g = e * count + a:
 * counts / offsets have E * count (+1) entries, and the capacity is
 * T*k + min(E * count, T*k) * (BLOCK_M - 1) (moe_lora_multi_pool_capacity).
 * A pool built by build_pool_multi serves only the *_multi calls with the
 * same adapters.  count = 1 with offsets {0, T} is exactly the single-adapter
 * path.
 * ------------------------------------------------------------------------ */
#define MOE_MAX_ADAPTERS 64

/* offsets: HOST int32 array of count + 1 entries, 0 = offsets[0] <= ... <=
 * offsets[count] = T (else MOE_ERR_INVALID); 1 <= count <= MOE_MAX_ADAPTERS
 * (more: MOE_ERR_UNSUPPORTED).  Read during the call only. */
typedef struct moe_adapters {
  int32_t count;
  const int32_t* offsets;
} moe_adapters;

moe_status moe_lora_multi_pool_capacity(const moe_lora_desc* desc, const moe_adapters* adapters,
                                        int64_t* rows);
moe_status moe_lora_multi_workspace_size(const moe_lora_desc* desc, const moe_adapters* adapters,
                                         size_t* saved_bytes, size_t* scratch_bytes);
/* build_pool with (expert, adapter) groups: counts [E*count], offsets
 * [E*count + 1]; rows of a group follow ascending route index. */
moe_status build_pool_multi(const moe_lora_desc* desc, const moe_adapters* adapters, const int32_t* topk_idx,
                            int32_t* counts, int32_t* offsets, int32_t* route_to_row, int32_t* row_to_route,
                            int64_t capacity, int32_t* device_error, void* stream);
/* moe_lora_forward / moe_lora_backward over the roots (adapters != NULL). */
moe_status moe_lora_forward_multi(const moe_lora_desc* desc, const moe_adapters* adapters, const moe_pool* pool,
                                  const void* x, const float* topk_w, const moe_lora_params* params, void* out,
                                  void* saved, size_t saved_bytes, void* scratch, size_t scratch_bytes,
                                  void* stream);
moe_status moe_lora_backward_multi(const moe_lora_desc* desc, const moe_adapters* adapters, const moe_pool* pool,
                                   const void* grad_out, const float* topk_w, const moe_lora_params* params,
                                   const void* saved, size_t saved_bytes, void* grad_x, float* grad_topk_w,
                                   const moe_lora_grads* grads, void* scratch, size_t scratch_bytes,
                                   void* stream);

/* Optional per-kernel timing (the pages' backward carries an optional kernel
 * trace: PR #9 review-bot Overview).  When enabled, every kernel the library
 * launches is bracketed by two HIP events recorded on its launch stream; the
 * events are created on first use and reused.  Off by default.
 *   moe_lora_trace_enable(1 / 0)  turn recording on / off (process-wide)
 *   moe_lora_trace_collect()      wait for the recorded events and add their
 *                                 elapsed times to per-kernel totals
 *   moe_lora_trace_count()        number of kernels with totals
 *   moe_lora_trace_entry(i, ...)  name (static storage until the next reset),
 *                                 launch count and total milliseconds of entry i
 *   moe_lora_trace_reset()        clear the totals */
void moe_lora_trace_enable(int32_t on);
moe_status moe_lora_trace_collect(void);
int32_t moe_lora_trace_count(void);
moe_status moe_lora_trace_entry(int32_t i, const char** name, int64_t* launches, double* total_ms);
void moe_lora_trace_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* MOELORA_H */
