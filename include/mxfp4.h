/*
 * mxfp4.h - C ABI of libmxfp4.so: fused MXFP4 dequantize-and-multiply on
 * AMD Instinct MI355X (gfx950).
 *
 * Weight format (OCP MX FP4), as stored by the pages this implements
 * ("cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs": module doc, DECODE and
 * PEROP shaders, MoeBankCodec::lens):
 *   A rows x cols tensor (cols % 32 == 0) is rows*cols/2 code bytes followed
 *   by rows*cols/32 scale bytes, rows*cols*17/32 bytes in all.
 *   - Code plane, row-major: element (r, c) is nibble c&1 (low nibble first)
 *     of byte (r*cols + c)/2.  A code n is E2M1: (-1)^(n>>3) times
 *     {0, 0.5, 1, 1.5, 2, 3, 4, 6}[n & 7] (code 8 is -0).
 *   - Scale plane, row-major: byte r*(cols/32) + c/32 is the E8M0 scale k of
 *     the 32-element group holding (r, c): 2^(k-127); k = 255 is NaN and
 *     k = 0 is 2^-127.
 *   - The weight is the E2M1 value times its scale.
 *
 * Conventions for every entry point:
 *   - Pointers named w, gate, up, down, x, y, out, workspace are DEVICE
 *     pointers owned by the caller and must be 16-byte aligned; logits,
 *     topk_ids, topk_w and the grouping arrays are device pointers, 4-byte
 *     aligned.
 *   - stream is a hipStream_t (NULL = the default stream).  Calls enqueue
 *     kernels on it and return: no host synchronisation, no allocation, no
 *     pointer kept after return.
 *   - Arguments are checked on the host before anything is launched.  On
 *     failure nothing is launched and a negative status is returned; the
 *     message is available from mxfp4_last_error() (per thread).
 *   - There is no CPU fallback: every result is computed by HIP kernels.
 *   - Activations/outputs are row-major: x [b][cols], y [b][rows].
 *   - Accuracy: weights are decoded exactly; fp32 activations enter the
 *     matrix cores as two bf16 parts, hi = x truncated to bf16 and
 *     lo = nearest bf16 of x - hi (|x - hi - lo| < 2^-15 |x|; any finite x,
 *     up to the fp32 maximum); accumulation is fp32.  Every output is within
 *     1e-4 * sum_c |W[r][c] * x[c]| of the exact product.  A NaN activation
 *     or scale gives NaN outputs; an infinite fp32 activation gives NaN for
 *     every output of its token (its low part is inf - inf).
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MXFP4_OK 0
#define MXFP4_EINVAL (-1)     /* bad size, dtype, null pointer or out-of-range argument */
#define MXFP4_EALIGN (-2)     /* a pointer is not aligned as documented */
#define MXFP4_EWORKSPACE (-3) /* workspace smaller than the size query returned */
#define MXFP4_ELAUNCH (-4)    /* the HIP runtime refused a launch */

/* Element types of activations and outputs. */
#define MXFP4_F32 0
#define MXFP4_BF16 1

/* Largest accepted sizes (checked; larger calls return MXFP4_EINVAL). */
#define MXFP4_MAX_ROWS (1 << 24)
#define MXFP4_MAX_COLS (1 << 14)
#define MXFP4_MAX_TENSOR_BYTES ((int64_t)1 << 31) /* one rows x cols tensor */
#define MXFP4_MAX_TOKENS (1 << 20)
#define MXFP4_MAX_EXPERTS 1024
#define MXFP4_MAX_TOP_K 32

/* Byte size of a rows x cols tensor, rows*cols*17/32; -1 if cols % 32 != 0
 * or a size is negative.  Host only. */
int64_t mxfp4_nbytes(int64_t rows, int64_t cols);

/* Dequantize W (rows x cols) to out [rows][cols] of out_dtype (MXFP4_F32 or
 * MXFP4_BF16).  Bit-exact: every finite weight is exactly representable in
 * both types; overflow gives +-inf; a scale-255 group gives 0x7FC00000
 * (fp32) / 0x7FC0 (bf16) for every element.  Follows the DECODE shader
 * (mx_e2m1, mx_e8m0) of "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs".
 * rows >= 1, cols >= 32. */
int mxfp4_dequant(const void *w, int64_t rows, int64_t cols, void *out, int out_dtype,
                  void *stream);

/* Decode matvec: y[r] = sum_c W[r][c] * x[c], fp32 in and out.
 * "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs", matmat with b = 1
 * (mxfp4_mv).  Same kernel and same result, bit for bit, as mxfp4_gemm
 * with b = 1. */
int mxfp4_matvec(const void *w, int64_t rows, int64_t cols, const float *x, float *y,
                 void *stream);

/* Small-batch GEMM: y[t][r] = sum_c W[r][c] * x[t][c] for t < b.
 * x is [b][cols] of x_dtype, y is [b][rows] of y_dtype (fp32 accumulate).
 * "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs", matmat (mxfp4_mm).
 * Each token's row equals, bit for bit, what the same call gives for that
 * token alone.  b >= 1. */
int mxfp4_gemm(const void *w, int64_t rows, int64_t cols, const void *x, int x_dtype, int64_t b,
               void *y, int y_dtype, void *stream);

/* MXFP8 quantization of activations, the activation side of
 * mxfp4_gemm_a8 (the OCP MX family that "cortiq-engine 0.8.40,
 * src/gpu_wgpu/mxfp4.rs" names in its module doc, with E4M3 elements):
 * for each block of 32 consecutive elements of a row of x [b][cols]
 * (x_dtype MXFP4_F32 or MXFP4_BF16, cols % 32 == 0), with a = the block's
 * largest magnitude, the shared exponent E = floor(log2 a) - 8 is stored as
 * the byte E + 127 clamped to [0, 254] in s [b][cols/32], and each element
 * becomes the E4M3 code (sign bit 7, exponent bias 7, 3 mantissa bits,
 * largest finite 448) nearest to x / 2^E, ties to even, magnitudes above
 * 448 saturating to 448, in q [b][cols].  A block of zeros gives the byte 0
 * and zero codes; a block holding NaN or an infinity gives 255 (NaN) and
 * zero codes.  x, q 16-byte aligned. */
int mxfp8_quantize(const void *x, int x_dtype, int64_t b, int64_t cols, uint8_t *q, uint8_t *s,
                   void *stream);

/* Workspace bytes of mxfp4_gemm_a8 (the quantized activations); 0 on bad
 * sizes (cols must be a multiple of 128). */
size_t mxfp4_gemm_a8_workspace_size(int64_t b, int64_t cols);

/* Opt-in block-scaled FP4 x FP8 GEMM: y[t][r] = sum_c W[r][c] * xq[t][c],
 * where xq is x quantized to MXFP8 (mxfp8_quantize), on the CDNA4
 * block-scaled matrix instruction v_mfma_scale_f32_16x16x128_f8f6f4: the
 * weights enter as stored (E2M1 codes with their E8M0 scales), the
 * activations as E4M3 with theirs, no decode.  Accuracy (its own contract,
 * not the 1e-4 rule of mxfp4_gemm): within 2^-7 * sum_c |W[r][c] *
 * xq[t][c]| of the exact product with the quantized activations (the
 * matrix core adds 32-element blocks exactly but aligns the products inside
 * a block to the block's largest); against the unquantized x the MXFP8
 * rounding adds up to 2^-4 of each element (1/8 for a block's largest when
 * it saturates).  Worth it where a product is a dense contraction (tens of
 * tokens and more).  cols % 128 == 0; x [b][cols] of x_dtype; y [b][rows]
 * of y_dtype; workspace at least mxfp4_gemm_a8_workspace_size(b, cols)
 * bytes, 16-byte aligned, scratch owned by the call until the stream
 * reaches it.  Errors as mxfp4_gemm, MXFP4_EWORKSPACE for a short
 * workspace. */
int mxfp4_gemm_a8(const void *w, int64_t rows, int64_t cols, const void *x, int x_dtype,
                  int64_t b, void *y, int y_dtype, void *workspace, size_t workspace_bytes,
                  void *stream);

/* Stable grouping of routed pairs by expert (the first step of the expert
 * bank), exposed for callers and tests.  Pairs are p = t*top_k + k.
 *   offsets [n_experts+1]: pairs of expert e occupy slots
 *       offsets[e] .. offsets[e+1]-1, in increasing p;
 *   pair_of_slot [n_tokens*top_k]: the pair in each slot;
 *   slot_of_pair [n_tokens*top_k]: the slot of each pair, -1 for a pair
 *       whose id is outside [0, n_experts) (such a pair is dropped).
 * "rlx-cpu 0.2.17, src/gguf_matmul.rs", grouped_moe_sort_plan. */
int moe_route_group(const int32_t *topk_ids, int64_t n_tokens, int64_t top_k, int64_t n_experts,
                    int32_t *offsets, int32_t *pair_of_slot, int32_t *slot_of_pair,
                    void *stream);

/* Device router: top-k experts of each token from its gating logits, and
 * renormalised route weights.  The pages give no router (their MoE frame,
 * "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs", takes the picks and weights
 * as inputs); this is the routing the 64-expert decode workload states:
 * softmax over the logits, the top_k most probable kept, their
 * probabilities renormalised to sum to 1.
 *   logits [n_tokens][n_experts] fp32 (device).
 *   topk_ids [n_tokens][top_k] (device): slot k holds the expert of rank k,
 *       ranks by descending logit; equal logits rank the lower index first;
 *       -0 equals +0; NaN ranks below every number.
 *   topk_w [n_tokens][top_k] fp32 (device): w_k = exp(l_k - l_0) /
 *       sum_j exp(l_j - l_0) over the chosen logits, l_0 the largest (equal
 *       to p_k / sum_j p_j of the full softmax); fp32 expf, summed in slot
 *       order.  Finite logits give finite weights; otherwise IEEE arithmetic
 *       of this formula (e.g. NaN when the largest is +inf).
 * 1 <= n_experts <= MXFP4_MAX_EXPERTS, 1 <= top_k <= min(MXFP4_MAX_TOP_K,
 * n_experts).  Pointers 4-byte aligned (MXFP4_EALIGN).  The output feeds
 * moe_experts_mxfp4 and moe_route_group directly. */
int moe_route_topk(const float *logits, int64_t n_tokens, int64_t n_experts, int64_t top_k,
                   int32_t *topk_ids, float *topk_w, void *stream);

/* Workspace bytes of moe_experts_mxfp4_a8 (0 on bad sizes: hidden and
 * inter must be multiples of 512). */
size_t moe_experts_mxfp4_a8_workspace_size(int64_t n_tokens, int64_t top_k, int64_t n_experts,
                                           int64_t hidden, int64_t inter);

/* Opt-in routed expert bank on the block-scaled FP4 x FP8 product, for
 * dense prefill experts: the bank of moe_experts_mxfp4 with x quantized to
 * MXFP8 (mxfp8_quantize) before gate/up, h = silu(g) * u computed in fp32
 * and quantized to MXFP8 before down, and every expert product on
 * v_mfma_scale_f32_16x16x128_f8f6f4 (weights as stored, no decode).
 * Accuracy (its own contract, that of mxfp4_gemm_a8 for each product): each
 * of g, u, y within 2^-7 of the sum of |w * a| over its terms of the exact
 * product with its quantized activation a (xq for g and u, hq for y), then
 * out[t] = sum_k topk_w[p] * y_p in slot order, fp32, rounded to out_dtype;
 * against the unquantized x and h, the MXFP8 rounding adds up to 2^-4 of
 * each element.  The same routing, grouping and combine as
 * moe_experts_mxfp4 (ids outside [0, n_experts) drop the pair), items of up
 * to 64 tokens per expert.  hidden % 512 == 0, inter % 512 == 0; other
 * arguments, layout and errors as moe_experts_mxfp4; the workspace (device,
 * 16-byte aligned, at least moe_experts_mxfp4_a8_workspace_size bytes) is
 * scratch owned by the call until the stream reaches it.
 * "cortiq-engine 0.8.77, src/qtensor/moe_fast.rs" (gate_up_block,
 * down_block); "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs" (module doc:
 * the OCP MX formats). */
int moe_experts_mxfp4_a8(const void *gate, const void *up, const void *down, int64_t n_experts,
                         int64_t hidden, int64_t inter, const void *x, int x_dtype,
                         int64_t n_tokens, const int32_t *topk_ids, const float *topk_w,
                         int64_t top_k, void *out, int out_dtype, void *workspace,
                         size_t workspace_bytes, void *stream);

/* Workspace bytes moe_experts_mxfp4 needs for these sizes (0 on bad sizes). */
size_t moe_experts_mxfp4_workspace_size(int64_t n_tokens, int64_t top_k, int64_t n_experts,
                                        int64_t hidden, int64_t inter, int x_dtype);

/* Routed expert bank.  For each token t and slot k (pair p = t*top_k + k)
 * with expert e = topk_ids[p]:
 *     g = W_gate[e] x_t,  u = W_up[e] x_t        (W_gate, W_up: inter x hidden)
 *     h = silu(g) * u,  silu(g) = g / (1 + e^-g)
 *     y_p = W_down[e] h                          (W_down: hidden x inter)
 *     out[t] = sum_k topk_w[p] * y_p             (in slot order, fp32)
 * gate, up, down: n_experts tensors each, contiguous, stride
 * mxfp4_nbytes(rows, cols) (which must be a multiple of 16).
 * x [n_tokens][hidden] of x_dtype; out [n_tokens][hidden] of out_dtype.
 * The activation h is kept in x_dtype (rounded to bf16, nearest-even, when
 * x is bf16); accumulation is fp32.  Each expert's weights are streamed
 * once per call for all of its tokens.  Ids outside [0, n_experts) drop the
 * pair.  The workspace (device, 16-byte aligned, at least
 * moe_experts_mxfp4_workspace_size bytes) is scratch owned by the call
 * until the stream reaches it; it needs no initialisation.
 * "cortiq-engine 0.8.77, src/qtensor/moe_fast.rs" (gate_up_block,
 * down_block); "cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs"
 * (dsv4_global_gate_up_mxfp4, dsv4_global_down_mxfp4, generic f32
 * weighting, mxg_bf16 rounding); "rlx-cpu 0.2.17, src/gguf_matmul.rs"
 * (grouped_moe_sort_plan, grouped_moe_unpermute_out). */
int moe_experts_mxfp4(const void *gate, const void *up, const void *down, int64_t n_experts,
                      int64_t hidden, int64_t inter, const void *x, int x_dtype, int64_t n_tokens,
                      const int32_t *topk_ids, const float *topk_w, int64_t top_k, void *out,
                      int out_dtype, void *workspace, size_t workspace_bytes, void *stream);

/* moe_experts_mxfp4 with each expert's tensors anywhere the GPU can read:
 * gate, up and down are tables of n_experts pointers (device arrays, 8-byte
 * aligned), entry e pointing to expert e's tensor (16-byte aligned, the
 * stored two-plane layout) in device memory or in pinned host memory mapped
 * into the device address space (hipHostMalloc).  This serves the experts a
 * card's memory does not hold ("cortiq-engine 0.8.77, src/qtensor/
 * moe_fast.rs", module contract; "cortiq-engine 0.8.40,
 * src/gpu_wgpu/mxfp4.rs", global_bank_case's cold winner): the same kernels
 * read a host-resident expert's weights over the host link, once per work
 * item, with no copy into device memory and no CPU arithmetic.  Results
 * equal moe_experts_mxfp4's on the same weights bit for bit.  The table
 * entries are device data and are not checked: each must be a valid,
 * device-accessible pointer to a tensor of the stated shape.  Other
 * arguments, workspace and errors as moe_experts_mxfp4 (workspace size from
 * moe_experts_mxfp4_workspace_size). */
int moe_experts_mxfp4_ptrs(const void *const *gate, const void *const *up,
                           const void *const *down, int64_t n_experts, int64_t hidden,
                           int64_t inter, const void *x, int x_dtype, int64_t n_tokens,
                           const int32_t *topk_ids, const float *topk_w, int64_t top_k,
                           void *out, int out_dtype, void *workspace, size_t workspace_bytes,
                           void *stream);

/* The address at which kernels on the current device read the memory at p:
 * p itself for device memory, the mapped address for pinned host memory
 * (hipHostMalloc).  Host only (a runtime query, no allocation).  Returns
 * MXFP4_EINVAL for pageable host memory or any pointer the runtime does not
 * know, which no kernel may be given.  For building the tables of
 * moe_experts_mxfp4_ptrs. */
int mxfp4_device_address(const void *p, void **device_ptr);

/* moe_experts_mxfp4 for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and result, bit for bit, with no workspace argument and no
 * allocation of any kind.  The scratch it needs lives in a static device
 * array of MXFP4_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held
 * until the process ends; its address is looked up on the first call on
 * each device (that device current).  Sizes whose workspace query exceeds
 * MXFP4_NOALLOC_SCRATCH_BYTES are refused with MXFP4_EWORKSPACE before
 * anything is launched (the 64-expert decode layer needs about 1.2 MB; a
 * 512-token prefill of 7168 x 2048 experts at top 8 needs 134 MB and does
 * not fit).  Every call on a GPU uses that GPU's one array: calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  The scratch needs no clearing between calls
 * (every call writes each part before reading it).  Other errors as
 * moe_experts_mxfp4. */
#define MXFP4_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_experts_mxfp4_noalloc(const void *gate, const void *up, const void *down,
                              int64_t n_experts, int64_t hidden, int64_t inter, const void *x,
                              int x_dtype, int64_t n_tokens, const int32_t *topk_ids,
                              const float *topk_w, int64_t top_k, void *out, int out_dtype,
                              void *stream);

/* Stage-isolation variant of moe_experts_mxfp4 (the gs_in / gs_out hooks of
 * "cortiq-engine 0.8.77, src/qtensor/moe_fast.rs", run_stages).  h is in
 * SLOT order ([n_tokens*top_k][inter] of x_dtype, slot as returned by
 * moe_route_group); pairs with slot -1 have no row.
 *   h_out != NULL: after gate/up + SwiGLU, copy h there.
 *   h_in != NULL : skip gate/up and run down + combine on h_in.
 *   out may be NULL when only h_out is wanted. */
int moe_experts_mxfp4_stages(const void *gate, const void *up, const void *down,
                             int64_t n_experts, int64_t hidden, int64_t inter, const void *x,
                             int x_dtype, int64_t n_tokens, const int32_t *topk_ids,
                             const float *topk_w, int64_t top_k, void *out, int out_dtype,
                             void *workspace, size_t workspace_bytes, const void *h_in,
                             void *h_out, void *stream);

/* V4.1 expert bank ("cortiq-engine 0.8.40, src/gpu_wgpu/mxfp4.rs":
 * dsv4_global_gate_up_mxfp4 and dsv4_global_down_mxfp4 with their bf16
 * flag, and the host expert of global_bank_case).  x and out are bf16.  For
 * each routed pair p = (t, k), e = topk_ids[p], w = topk_w[p]:
 *     g = bf16(W_gate[e] x_t),  u = bf16(W_up[e] x_t)   (fp32 products rounded)
 *     if swiglu_limit > 0:  u = clamp(u, -limit, limit),  g = min(g, limit)
 *     h_p = bf16(w * (silu(g) * u))                     (route weight folded in)
 *     out[t] = bf16(sum over the token's slots of W_down[e] h_p)   (no weight)
 * swiglu_limit: finite, >= 0; 0 means no limit.  has_shared = 1 applies one
 * more expert, index n_experts, to every token with weight 1 as slot top_k:
 * gate, up and down then hold n_experts + 1 tensors each, the shared one
 * last, and top_k + has_shared <= MXFP4_MAX_TOP_K (the shared expert takes a
 * slot of its own; the workspace size query returns 0 and the call
 * MXFP4_EINVAL above that).  Ids outside [0, n_experts) drop the pair (they never select the
 * shared expert).  Summation order and accumulation as in moe_experts_mxfp4;
 * the down outputs of a token's slots are summed in slot order in fp32 and
 * rounded once.  Workspace: at least moe_experts_mxfp4_v41_workspace_size
 * bytes (device, 16-byte aligned, scratch owned by the call until the stream
 * reaches it).  Errors as moe_experts_mxfp4; also MXFP4_EINVAL for a
 * negative or non-finite limit or has_shared outside {0, 1}. */
size_t moe_experts_mxfp4_v41_workspace_size(int64_t n_tokens, int64_t top_k, int64_t n_experts,
                                            int64_t hidden, int64_t inter, int has_shared);
int moe_experts_mxfp4_v41(const void *gate, const void *up, const void *down, int64_t n_experts,
                          int64_t hidden, int64_t inter, const void *x, int64_t n_tokens,
                          const int32_t *topk_ids, const float *topk_w, int64_t top_k,
                          float swiglu_limit, int has_shared, void *out, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Stage-isolation variant of moe_experts_mxfp4_v41, as
 * moe_experts_mxfp4_stages: h in SLOT order, bf16,
 * [n_tokens * (top_k + has_shared)][inter]. */
int moe_experts_mxfp4_v41_stages(const void *gate, const void *up, const void *down,
                                 int64_t n_experts, int64_t hidden, int64_t inter, const void *x,
                                 int64_t n_tokens, const int32_t *topk_ids, const float *topk_w,
                                 int64_t top_k, float swiglu_limit, int has_shared, void *out,
                                 void *workspace, size_t workspace_bytes, const void *h_in,
                                 void *h_out, void *stream);

/* Message of the last failed call on this thread ("" if none). */
const char *mxfp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
