/*
 * lce.h -- C ABI of the MI355X (gfx950) fused linear cross-entropy library (liblce.so).
 *
 * The operations follow three pages:
 *   [P1] "Fused Linear Cross-Entropy: The Math, the Memory Wall, and Two Ways Around It"
 *   [P2] "Cut Cross Entropy visualized"
 *   [P3] "Greyhound -- Cross-Entropy"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor argument is a DEVICE pointer owned by the caller.  The library never
 *    allocates device memory and keeps no state between calls (apart from a per-device
 *    cache of the compute-unit count); scratch space is the caller's `workspace` buffer,
 *    sized by the matching *_workspace_bytes function.
 *  - Layouts are dense row-major: hidden [BT, H], W [V, H] (nn.Linear layout, [P1] "The
 *    setting"), logits [B, V]; targets are int64.  Tensor pointers and the workspace must
 *    be 16-byte aligned.  H must be a multiple of 8.  Vocabulary sizes and target ids are
 *    below 2^31 (targets are compared as 32-bit ids on the device).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL means the default stream) and is
 *    asynchronous: outputs are valid once the stream has completed.  Nothing is copied
 *    to the host unless LCE_FLAG_CHECK_TARGETS is given.
 *  - Errors are returned, never thrown.  Argument errors (LCE_ERR_NULL .. LCE_ERR_ARG)
 *    are detected on the host before any device work is enqueued; in that case no
 *    output is touched.
 *  - Identical inputs give identical output bits: every cross-workgroup reduction has a
 *    fixed order and no floating-point atomics are used.
 */
#ifndef LCE_H_
#define LCE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
/* The enums are int-sized in C; in C++ their underlying type is fixed to int as well, so that
 * any int a caller passes (an invalid dtype, say) is a value of the type and is rejected with
 * an error code rather than being undefined. */
#define LCE_ENUM_BASE : int
#else
#define LCE_ENUM_BASE
#endif

typedef enum lce_status LCE_ENUM_BASE {
  LCE_OK = 0,
  LCE_ERR_NULL = 1,         /* a required pointer is NULL */
  LCE_ERR_SHAPE = 2,        /* a size is out of range (negative, V < 1, H not a multiple of 8, ...) */
  LCE_ERR_DTYPE = 3,        /* dtype not supported by this entry point */
  LCE_ERR_ALIGNMENT = 4,    /* a tensor or workspace pointer is not 16-byte aligned */
  LCE_ERR_WORKSPACE = 5,    /* workspace_bytes smaller than the *_workspace_bytes requirement */
  LCE_ERR_ARG = 6,          /* bad scalar argument (reduction, z_loss_mult < 0 or NaN, grad_b without bias) */
  LCE_ERR_TARGET_RANGE = 7, /* (check mode only) a target is neither ignore_index nor in [0, V) */
  LCE_ERR_HIP = 8,          /* a HIP runtime call or kernel launch failed */
  LCE_ERR_SCRATCH_LIMIT = 9 /* (no-allocation entry point) the size exceeds its fixed scratch */
} lce_status;

typedef enum lce_dtype LCE_ENUM_BASE {
  LCE_DTYPE_F32 = 0,
  LCE_DTYPE_BF16 = 1,
  LCE_DTYPE_F16 = 2   /* IEEE half: lce_ce_with_grad_inplace only */
} lce_dtype;

typedef enum lce_reduction LCE_ENUM_BASE {
  LCE_REDUCTION_MEAN = 0, /* loss and grads scaled by 1 / max(n_valid, 1) */
  LCE_REDUCTION_SUM = 1   /* unscaled */
} lce_reduction;

/* Synchronise `stream` after the target pre-pass and return LCE_ERR_TARGET_RANGE if any
 * target is neither ignore_index nor a vocabulary id.  Without it such rows are treated
 * as ignored (no loss, zero gradient) and the call still returns LCE_OK. */
#define LCE_FLAG_CHECK_TARGETS 1u
/* grad_W is float32 [V, H] for bf16 inputs (rounded once from the fp32 accumulators instead
 * of to bf16).  In the chunked entry points the sum over the token chunks is kept in it
 * directly, so their workspace needs no fp32 accumulator of its own. */
#define LCE_FLAG_GRAD_W_FP32 2u
/* (lce_fwd_bwd_filtered only) vocabulary sorting before gradient filtering ("Cut Cross
 * Entropy visualized", "Vocabulary Sorting"): the vocabulary is ordered by each entry's
 * average logit over the rows that count (W . mean hidden row + b; ties by id), the call
 * runs on sorted copies of W, the bias and the targets, so the filter's tiles group
 * entries of similar average logit, and grad_W / grad_b are written in the original order.
 * The workspace then also holds the sorted copy of W (lce_fwd_bwd_workspace_bytes with this
 * flag); BT and V at most 2^24. */
#define LCE_FLAG_SORT_VOCAB 4u

/* Number of device kernels one lce_fwd_bwd call may launch (for lce_fwd_bwd_profiled). */
#define LCE_NUM_STAGES 7

/*
 * lce_fwd_bwd -- fused linear cross-entropy, forward and backward in one call.
 *
 * Computes z_t = W . hidden[t] + b for every token without materialising the [BT, V]
 * logits ([P1] "The setting"; [P2] "Forward Kernel"), the loss
 *     L = c * sum_{t : y_t != ignore_index} ( LSE(z_t) - z_t[y_t] + z_loss_mult * LSE(z_t)^2 )
 * with c = 1 / max(n_valid, 1) for LCE_REDUCTION_MEAN and c = 1 for LCE_REDUCTION_SUM
 * ([P1] "The setting"; z-loss term from [P3] opening formulas), and its gradients
 *     dlogits[t, :] = c * valid_t * ( softmax(z_t) * (1 + 2 * z_loss_mult * LSE(z_t)) - onehot(y_t) )
 *     grad_input    = dlogits . W,     grad_W = dlogits^T . hidden,     grad_b = sum_t dlogits[t, :]
 * ([P1] "The identity that makes fused fwbw possible" and "From dlogits to grad_input
 * and grad_W"; [P3] "Kernel design" for the z-loss factor).
 *
 * Arguments
 *   hidden      [BT, H] in `dtype`.                     W      [V, H] in `dtype`.
 *   bias        [V] in `dtype`, or NULL for no bias.  An entry of -inf masks its vocabulary
 *               entry: e^-inf = 0 in every sum, its dlogits and its rows of grad_W and grad_b
 *               are 0 (a counted target must not be masked).
 *   targets     [BT] int64; ignore_index marks rows that contribute nothing.
 *   BT >= 0, 8 <= H <= 2^20 with H a multiple of 8, V >= 1.
 *   dtype       LCE_DTYPE_BF16 or LCE_DTYPE_F32 (arithmetic: products accumulated in fp32;
 *               softmax statistics in fp32; bf16 dlogits operands rounded to nearest even).
 *   ignore_index  target value of ignored rows (usually -100).
 *   z_loss_mult   >= 0; 0 disables the z-loss term.
 *   reduction   LCE_REDUCTION_MEAN or LCE_REDUCTION_SUM.
 *   flags       0, LCE_FLAG_CHECK_TARGETS and/or LCE_FLAG_GRAD_W_FP32.
 *   loss_out    device float[1]: the loss L.                          (required)
 *   grad_input  device [BT, H] in `dtype`, fully overwritten, or NULL to skip it.
 *   grad_W      device [V, H] in `dtype` (float32 with LCE_FLAG_GRAD_W_FP32), fully
 *               overwritten, or NULL to skip it.
 *   grad_b      device [V] in `dtype`, fully overwritten, or NULL; must be NULL when bias is NULL.
 *   n_valid_out device int64[1]: number of rows with y != ignore_index, or NULL.
 *   lse_out     device float[BT]: LSE(z_t) per row (the statistic the backward reuses,
 *               [P2] "Breakdown: Backward Pass"), or NULL.
 *   workspace   device scratch of at least lce_fwd_bwd_workspace_bytes(BT, H, V, dtype, flags)
 *               bytes; contents on entry are ignored and on exit undefined.
 *   stream      hipStream_t to enqueue on.
 */
lce_status lce_fwd_bwd(const void* hidden, const void* W, const void* bias, const int64_t* targets,
                       int64_t BT, int64_t H, int64_t V, lce_dtype dtype, int64_t ignore_index,
                       float z_loss_mult, lce_reduction reduction, uint32_t flags, float* loss_out,
                       void* grad_input, void* grad_W, void* grad_b, int64_t* n_valid_out,
                       float* lse_out, void* workspace, size_t workspace_bytes, void* stream);

/* Same as lce_fwd_bwd; in addition, when ev_start/ev_stop are non-NULL arrays of
 * LCE_NUM_STAGES hipEvent_t handles created by the caller, records ev_start[k] and
 * ev_stop[k] on `stream` around the launch of stage k (names: lce_stage_name).  Stages
 * that a call does not launch get no records.  For per-kernel timing by benchmarks. */
lce_status lce_fwd_bwd_profiled(const void* hidden, const void* W, const void* bias,
                                const int64_t* targets, int64_t BT, int64_t H, int64_t V,
                                lce_dtype dtype, int64_t ignore_index, float z_loss_mult,
                                lce_reduction reduction, uint32_t flags, float* loss_out,
                                void* grad_input, void* grad_W, void* grad_b, int64_t* n_valid_out,
                                float* lse_out, void* workspace, size_t workspace_bytes,
                                void* stream, void* const* ev_start, void* const* ev_stop);

/*
 * lce_fwd_bwd_filtered -- lce_fwd_bwd with gradient filtering ("Cut Cross Entropy
 * visualized", "Gradient Filtering"): a lossy mode, off in every exact path.
 *
 * The gradient GEMMs consume the dlogits in tiles; a tile whose entries are all below
 * filter_eps in magnitude contributes nothing to the gradient it feeds (its MFMA work is
 * skipped, and for grad_W its share of grad_b is dropped too).  The tiles are
 *   grad_input: R tokens x C vocabulary entries (aligned at token 0, vocabulary entry 0);
 *   grad_W, grad_b: R vocabulary entries x C tokens,
 * with (R, C) = (256, 64) where the bf16 backward runs on the stored-operand GEMM (from
 * H = 1024, when its one-pass plan fits the workspace) and (64, 16) otherwise:
 * lce_filter_tile_shape gives them.
 * The test applies to the dlogits of the summed loss, valid * (softmax * (1 + 2 mu LSE) -
 * onehot), i.e. before the 1/n_valid of the mean, so it does not depend on the batch size.
 * The loss, n_valid and LSE are exact.  The gradients differ from lce_fwd_bwd's by the
 * dropped entries only (each below filter_eps times the reduction scale).
 *   filter_eps     >= 0 and finite; 0 disables filtering (the call is then lce_fwd_bwd).
 *   filter_counts  device int64[4] or NULL: skipped and examined tiles of the grad_input
 *                  pass, then of the grad_W pass (overwritten; only when filter_eps > 0).
 * flags: as lce_fwd_bwd, plus LCE_FLAG_SORT_VOCAB.
 * Other arguments, errors and workspace as lce_fwd_bwd (LCE_ERR_ARG for a bad filter_eps).
 */
lce_status lce_fwd_bwd_filtered(const void* hidden, const void* W, const void* bias,
                                const int64_t* targets, int64_t BT, int64_t H, int64_t V,
                                lce_dtype dtype, int64_t ignore_index, float z_loss_mult,
                                lce_reduction reduction, uint32_t flags, float* loss_out,
                                void* grad_input, void* grad_W, void* grad_b, int64_t* n_valid_out,
                                float* lse_out, void* workspace, size_t workspace_bytes,
                                void* stream, float filter_eps, int64_t* filter_counts);

/* The filter tiles of lce_fwd_bwd_filtered for these sizes ("Cut Cross Entropy visualized",
 * "Gradient Filtering"): *rows = R and *cols = C as described there (host only, no device
 * work).  LCE_ERR_ARG for NULL outputs, invalid sizes or dtype. */
lce_status lce_filter_tile_shape(int64_t BT, int64_t H, int64_t V, lce_dtype dtype, int64_t* rows, int64_t* cols);

/* Exact number of workspace bytes lce_fwd_bwd needs for these sizes (its whole extra
 * device memory), or 0 if the sizes are invalid. */
size_t lce_fwd_bwd_workspace_bytes(int64_t BT, int64_t H, int64_t V, lce_dtype dtype, uint32_t flags);

/* Name of stage k of lce_fwd_bwd ("targets", "fwd_lse", "target_logit", "merge",
 * "loss", "bwd_dinput", "bwd_dweight"), or NULL if k is out of range. */
const char* lce_stage_name(int k);

/*
 * lce_ce_with_grad_inplace -- cross-entropy on existing logits, with dlogits written over
 * the logits in place ([P3] "Kernel design" and "Raw kernel helper").
 *
 * For each row i of logits [B, V]:  ce_i = LSE(x_i) - x_i[y_i];  z_i = LSE(x_i)^2.
 *   ce_sum_out  device float[1] = sum over valid rows of ce_i.
 *   z_sum_out   device float[1] = sum over valid rows of z_i if z_loss_mult != 0, else 0.
 *   n_valid_out device int64[1] = number of rows with y_i != ignore_index.
 * On return logits holds the gradient of ce_sum + z_loss_mult * z_sum:
 *   dlogits_i = valid_i * ( softmax(x_i) * (1 + 2 * z_loss_mult * LSE(x_i)) - onehot(y_i) ),
 * rounded to the logits' dtype; ignored rows are written as zeros.  A mean-reduced loss is
 * ce_sum / max(n_valid, 1) and its gradient is these dlogits times the same factor.
 *   logits      [B, V] in `dtype` (LCE_DTYPE_BF16, LCE_DTYPE_F16 or LCE_DTYPE_F32; the page's
 *               kernel takes float16, bfloat16 and float32 logits), read then overwritten; -inf
 *               entries (masked, never a counted target) add nothing and get dlogit 0.
 *   targets     [B] int64.   B >= 0, V >= 1.   z_loss_mult >= 0.
 *   workspace   >= lce_ce_workspace_bytes(B, V, dtype) bytes.
 * Targets outside [0, V) that are not ignore_index are treated as ignored.
 */
lce_status lce_ce_with_grad_inplace(void* logits, const int64_t* targets, int64_t B, int64_t V,
                                    lce_dtype dtype, int64_t ignore_index, float z_loss_mult,
                                    float* ce_sum_out, float* z_sum_out, int64_t* n_valid_out,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * lce_ce_with_grad_inplace_noalloc -- lce_ce_with_grad_inplace for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same computation and results, with no workspace argument.  Its
 * scratch (12 bytes per row) lives in a fixed device array of the library, 3 MiB on every GPU
 * the library runs on, held until the process ends; the call allocates nothing.
 *   B <= LCE_NOALLOC_MAX_ROWS, else LCE_ERR_SCRATCH_LIMIT (checked before any device work).
 *   Other arguments and errors as lce_ce_with_grad_inplace.
 * Every call on one GPU uses that GPU's one scratch array: calls that overlap in time on the
 * same GPU (different streams or threads without ordering between them) race and must not
 * be made.
 */
#define LCE_NOALLOC_MAX_ROWS 262144
lce_status lce_ce_with_grad_inplace_noalloc(void* logits, const int64_t* targets, int64_t B, int64_t V,
                                            lce_dtype dtype, int64_t ignore_index, float z_loss_mult,
                                            float* ce_sum_out, float* z_sum_out, int64_t* n_valid_out,
                                            void* stream);

/*
 * lce_stream_bandwidth -- a measurement helper, not part of the loss: streams `bytes` through
 * device memory with plain 16-byte accesses (mode 0: read src; 1: write dst; 2: copy src to
 * dst), so that the memory rate this device actually sustains can be timed beside
 * lce_ce_with_grad_inplace, the HBM-bound kernel.  In mode 0, dst is a 4-byte device scratch
 * word that is at most written.  bytes a multiple of 16, pointers 16-byte aligned; errors as
 * above (LCE_ERR_ARG for another mode).
 */
lce_status lce_stream_bandwidth(int mode, const void* src, void* dst, size_t bytes, void* stream);

/*
 * lce_fwd_bwd_chunked -- the same loss and gradients by the token-chunked composition
 * ("Fused Linear Cross-Entropy: The Math, the Memory Wall, and Two Ways Around It",
 * Strategy 1 and "The chunk-size trick"; "Greyhound -- Cross-Entropy", "Relationship to
 * Chunked Linear Loss").  bf16 only.
 *
 * Tokens are processed in chunks of cs rows, cs = 2 * next_pow2(ceil(BT / ceil(V / H)))
 * (capped at BT): the chunk's logits are written once to a bf16 buffer of cs x V entries in
 * the workspace, turned into dlogits in place by the standalone cross-entropy kernel, and
 * consumed by the two gradient products.  Nothing is recomputed (6 BT V H flops instead of
 * lce_fwd_bwd's 10), at the price of the chunk buffer and an fp32 grad_W sum in device memory
 * (V x H x 4 bytes, unless LCE_FLAG_GRAD_W_FP32).  Results agree with lce_fwd_bwd within the
 * bf16 tolerances; they differ in rounding because the dlogits pass through bf16 storage.
 *
 *   flags   0, LCE_FLAG_CHECK_TARGETS and/or LCE_FLAG_GRAD_W_FP32 (grad_W is float32 [V, H]).
 *   lse_out LSE per row, or NULL.
 * Other arguments as lce_fwd_bwd, with V <= 2^22; LCE_ERR_DTYPE for float32 inputs.  The workspace must hold
 * lce_fwd_bwd_chunked_workspace_bytes(BT, H, V, dtype, flags) bytes (0 for float32).
 */
size_t lce_fwd_bwd_chunked_workspace_bytes(int64_t BT, int64_t H, int64_t V, lce_dtype dtype, uint32_t flags);
lce_status lce_fwd_bwd_chunked(const void* hidden, const void* W, const void* bias, const int64_t* targets,
                               int64_t BT, int64_t H, int64_t V, lce_dtype dtype, int64_t ignore_index,
                               float z_loss_mult, lce_reduction reduction, uint32_t flags, float* loss_out,
                               void* grad_input, void* grad_W, void* grad_b, int64_t* n_valid_out,
                               float* lse_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * lce_rows_forward / lce_rows_backward -- per-row outputs of the LM head for RL-style use
 * ("Fused Linear Cross-Entropy: The Math, the Memory Wall, and Two Ways Around It",
 * Strategy 2 keeps each row's target log-probability and softmax entropy beside the LSE)
 * and the gradients of any per-row weighted sum of them.  bf16 only.  The forward is one pass
 * over the vocabulary with no logits stored (LSE and the softmax-weighted mean logit kept per
 * vocabulary tile from the fp32 accumulator, then merged per row; the tokens in as many
 * launches as the workspace needs).  The backward runs as lce_fwd_bwd's does, in vocabulary
 * blocks whose dlogits are formed once from per-token coefficients and feed both gradient
 * products, within the same one-chunk workspace; where that plan does not fit (tiny sizes) it is
 * the token-chunked composition of lce_fwd_bwd_chunked.
 *
 * For row t with z_t = W h_t + b, LSE_t = log sum_v exp(z_tv), p_t = softmax(z_t) and
 * valid_t = (y_t != ignore_index):
 *   row_loss[t] = valid_t (LSE_t - z_t[y_t] + z_loss_mult LSE_t^2)   (reduction 'none')
 *   logprobs[t] = valid_t (z_t[y_t] - LSE_t)
 *   entropy[t]  = LSE_t - sum_v p_tv z_tv                              (every row)
 * lce_rows_forward writes any of lse_out, logprobs_out, entropy_out, row_loss_out (device
 * float[BT] each, or NULL) and n_valid_out (int64[1] or NULL).
 * lce_rows_backward writes grad_input, grad_W, grad_b (as lce_fwd_bwd; each may be NULL) for
 *   F = sum_t grad_row_loss[t] row_loss[t] + grad_logprobs[t] logprobs[t] + grad_entropy[t] entropy[t]
 * (each upstream gradient a device float[BT], or NULL for zeros).  Its dlogits are
 *   p_tv (alpha_t + beta_t z_tv) - gamma_t [v == y_t],
 *   alpha_t = valid_t (gl_t (1 + 2 mu LSE_t) - gp_t) + ge_t E_p[z_t],  beta_t = -ge_t,
 *   gamma_t = valid_t (gl_t - gp_t).
 * lse_saved, entropy_saved: device float[BT] each, both or neither (else LCE_ERR_ARG): the LSE
 * and entropy that lce_rows_forward wrote for the same inputs.  With them, E_p[z] = LSE - entropy
 * is known and the dlogits come straight from the logits GEMM's fp32 accumulator; without them
 * the backward first recomputes LSE and entropy with the forward's pass (on the token-chunked
 * composition: from the chunk's bf16 logits).  Values that do not belong to these inputs give
 * gradients of no meaning (they are not checked).
 * flags: LCE_FLAG_CHECK_TARGETS; lce_rows_backward also LCE_FLAG_GRAD_W_FP32.  Workspace:
 * lce_rows_workspace_bytes, within one logits chunk of lce_fwd_bwd wherever the block plan fits
 * (otherwise the larger of lce_fwd_bwd_chunked_workspace_bytes plus 20 bytes per row and the
 * forward's per-(vocabulary tile, token) partials); one workspace serves both calls.  Errors
 * as lce_fwd_bwd_chunked.
 */
size_t lce_rows_workspace_bytes(int64_t BT, int64_t H, int64_t V, lce_dtype dtype, uint32_t flags);
lce_status lce_rows_forward(const void* hidden, const void* W, const void* bias, const int64_t* targets,
                            int64_t BT, int64_t H, int64_t V, lce_dtype dtype, int64_t ignore_index,
                            float z_loss_mult, uint32_t flags, float* lse_out, float* logprobs_out,
                            float* entropy_out, float* row_loss_out, int64_t* n_valid_out, void* workspace,
                            size_t workspace_bytes, void* stream);
lce_status lce_rows_backward(const void* hidden, const void* W, const void* bias, const int64_t* targets,
                             int64_t BT, int64_t H, int64_t V, lce_dtype dtype, int64_t ignore_index,
                             float z_loss_mult, uint32_t flags, const float* grad_row_loss,
                             const float* grad_logprobs, const float* grad_entropy, const float* lse_saved,
                             const float* entropy_saved, void* grad_input, void* grad_W, void* grad_b,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes lce_ce_with_grad_inplace needs (per-row partial results), or 0 if invalid. */
size_t lce_ce_workspace_bytes(int64_t B, int64_t V, lce_dtype dtype);

/* Human-readable text for a status code (static storage). */
const char* lce_status_string(lce_status s);

/* Library version string, e.g. "0.1.0 gfx950". */
const char* lce_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LCE_H_ */
