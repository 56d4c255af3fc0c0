/*
 * hc.h -- C ABI of libhc.so, the MI355X (gfx950) hyper-connection residual mix.
 *
 * The residual of a DeepSeek-V4.1 block is hc = 4 parallel streams of width d
 * (the released configuration; the page's split kernel and Block are written
 * for any stream count hc). Each sublayer is bracketed by: a projection of the
 * flattened streams to M = (2+hc)*hc mix numbers (24 at hc = 4), a split of
 * those numbers into collapse ("pre"),
 * output ("post") and combine ("comb") coefficients made nearly doubly
 * stochastic by Sinkhorn rounds, a collapse of the streams into the sublayer
 * input, and an expansion of the sublayer output back into the streams.
 *
 * Sources, cited by page title and section:
 *   atlas page "Block" -- code section: Block.forward, Block.hc_mixes,
 *       Block.hc_pre, Block.hc_post; parameter table.
 *   atlas page "Stream combination" -- summary, code section (the split and
 *       Sinkhorn kernel and its wrapper), released configuration.
 *   "DeepSeek-V4.1-Flash" diagram -- blocks "Mixing Coefficients", "sigma",
 *       "x + eps_hc", "2 sigma", "First Sinkhorn Round", "Sinkhorn Round",
 *       "Cast", "Single-Pass mHC", "Cast to MXFP8".
 *   "DeepSeek-R1 donor reference" -- RMSNorm passages.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or retains them. Tensors are dense and row-major.
 *     n is the number of tokens (batch * positions, flattened).
 *   - Layouts: streams [n][hc][d]; sublayer input/output [n][d];
 *     hc_fn [M][hc*d] fp32 with flat input index c = j*d + e;
 *     mixes [n][M] fp32 (pre logits (hc) | post logits (hc) | comb logits
 *     (hc*hc, row-major)); pre, post [n][hc] fp32; comb [n][hc][hc] fp32 where
 *     comb[j][k] weighs OLD stream j into NEW stream k; hc_scale [3], hc_base
 *     [M] fp32. M = (2+hc)*hc.
 *   - dtype selects the stream element type: HC_F32 or HC_BF16. Coefficients
 *     and parameters are always fp32. Arithmetic is fp32; bf16 results are
 *     rounded to nearest, ties to even.
 *   - Supported sizes: 1 <= hc <= 8; 8 <= d <= 1048576 and d % 8 == 0;
 *     0 <= n < 2^31 (n == 0 is a no-op returning HC_OK without touching any
 *     pointer) and n * d <= 2^40; and every kernel grid the call forms must
 *     fit a launch (at most 2^32 - 1 work-items): with four streams that is
 *     n < 2^28 and n * d <= 2^35, with other stream counts
 *     n * ceil(d / 512) < 2^26. Larger sizes return HC_ERR_SHAPE before any
 *     HIP call (hc_split_sinkhorn: n < 2^31 with four streams, n < 2^26
 *     otherwise). hc == 4 runs the
 *     single-pass kernels; other stream counts run one kernel per step (the
 *     fused boundary as expand, projection, split, collapse in sequence).
 *   - Alignment: every tensor pointer (streams, sublayer input/output, hc_fn,
 *     mixes, pre/post/comb and their _prev / pre_mix inputs, workspace) must be
 *     16-byte aligned; hc_scale and hc_base need 4-byte alignment.
 *   - stream is a hipStream_t passed as void* (NULL = default stream). Calls
 *     only enqueue work; they never synchronise the device.
 *   - All arguments are validated before any HIP call; on a validation error
 *     nothing is enqueued. HC_ERR_HIP reports a launch failure
 *     (hipGetLastError after the launch).
 *   - Outputs must not overlap inputs or each other, except where an entry
 *     point says an exact in-place alias is allowed (HC_ERR_ALIAS otherwise).
 *   - Entry points that take a workspace need at least hc_workspace_size(n, hc,
 *     d) bytes of device memory, 16-byte aligned, owned by the caller. Its
 *     contents on entry are irrelevant; concurrent calls must not share one.
 */
#ifndef HC_H
#define HC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HC_ABI_VERSION 1

#define HC_OK 0
#define HC_ERR_NULL (-1)        /* a required pointer is NULL */
#define HC_ERR_SHAPE (-2)       /* n < 0, d < 1 or n, d, n * d too large */
#define HC_ERR_UNSUPPORTED (-3) /* hc outside 1..8, d % 8 != 0, unknown dtype */
#define HC_ERR_ALIGN (-4)       /* a pointer breaks the alignment rule */
#define HC_ERR_ARG (-5)         /* sinkhorn_iters < 1, eps or norm_eps negative or not finite */
#define HC_ERR_ALIAS (-6)       /* outputs overlap inputs or each other */
#define HC_ERR_WORKSPACE (-7)   /* workspace missing or smaller than required */
#define HC_ERR_HIP (-8)         /* the HIP runtime reported an error */
#define HC_ERR_SCRATCH (-9)     /* hc_fused_step_noalloc: needs more than the static scratch */

/* Bytes of the static device scratch behind hc_fused_step_noalloc (per GPU). */
#define HC_NOALLOC_SCRATCH_BYTES (32u << 20)

#define HC_F32 0
#define HC_BF16 1

/* Version of this ABI (HC_ABI_VERSION of the built library). */
int hc_abi_version(void);

/* Static, human-readable name of a status code. Never NULL. */
const char* hc_status_string(int status);

/* Bytes of workspace hc_mixes and hc_fused_step need for (n, hc, d); 0 for
 * n == 0 or unsupported sizes. Depends on nothing but its arguments. */
size_t hc_workspace_size(int64_t n, int hc, int64_t d);

/*
 * Mix projection -- atlas "Block", Block.hc_mixes (first three statements);
 * diagram "Mixing Coefficients".
 * For each token the hc streams are flattened to D = hc*d values, and
 *   mixes[t][i] = (sum_c hc_fn[i][c] * x[t][c]) / sqrt(mean_c(x[t][c]^2) + norm_eps)
 * for i < M = (2+hc)*hc. One RMS statistic covers all hc*d values of the token.
 * The released configuration uses norm_eps = 1e-20.
 *   x     [n][hc][d] dtype      in
 *   hc_fn [M][hc*d] fp32        in
 *   mixes [n][M] fp32           out
 */
int hc_mixes(const void* x, int dtype, int64_t n, int hc, int64_t d, const float* hc_fn,
             float norm_eps, float* mixes, void* workspace, size_t workspace_bytes,
             void* stream);

/*
 * Split and Sinkhorn -- atlas "Stream combination", summary and code section;
 * diagram blocks "sigma", "x + eps_hc", "2 sigma", "First Sinkhorn Round",
 * "Sinkhorn Round".
 * With m = mixes[t], s = hc_scale, b = hc_base:
 *   pre[t][j]  = sigmoid(s[0]*m[j] + b[j]) + eps
 *   post[t][j] = 2 * sigmoid(s[1]*m[hc+j] + b[hc+j])
 *   comb[t]    = Sinkhorn(L), L[j][k] = s[2]*m[2hc+j*hc+k] + b[2hc+j*hc+k]:
 *     row softmax (max subtracted), + eps on every entry, divide each column by
 *     (column sum + eps); then sinkhorn_iters-1 rounds of: divide each row by
 *     (row sum + eps), divide each column by (column sum + eps).
 * Released configuration: sinkhorn_iters = 20, eps = 1e-6.
 *   mixes [n][M] in; pre [n][hc], post [n][hc], comb [n][hc][hc] out (fp32).
 */
int hc_split_sinkhorn(const float* mixes, const float* hc_scale, const float* hc_base,
                      int64_t n, int hc, int sinkhorn_iters, float eps, float* pre,
                      float* post, float* comb, void* stream);

/*
 * Collapse -- atlas "Block", Block.hc_pre.
 *   y[t][e] = sum_j pre_mix[t][j] * x[t][j][e]   (fp32 sum, one rounding to dtype)
 *   x [n][hc][d] dtype in; pre_mix [n][hc] fp32 in; y [n][d] dtype out.
 */
int hc_pre(const void* x, int dtype, const float* pre_mix, int64_t n, int hc, int64_t d,
           void* y, void* stream);

/*
 * Expand and combine -- atlas "Block", Block.hc_post.
 *   out[t][k][e] = post[t][k]*f[t][e] + sum_j comb[t][j][k]*residual[t][j][e]
 * (fp32 sum, one rounding to dtype). f and residual share dtype.
 *   f [n][d], residual [n][hc][d] in; post [n][hc], comb [n][hc][hc] in;
 *   out [n][hc][d] out. out == residual (exact in-place) is allowed.
 */
int hc_post(const void* f, const void* residual, int dtype, const float* post,
            const float* comb, int64_t n, int hc, int64_t d, void* out, void* stream);

/*
 * The sublayer RMSNorm of the collapsed input and its MXFP8 cast -- atlas
 * "Block", Block.forward (attn_norm / ffn_norm = RMSNorm(dim, norm_eps) on the
 * output of hc_pre); "DeepSeek-R1 donor reference", RMSNorm passages (scale by
 * 1/sqrt(mean x^2 + eps), multiply by the learned gain, restore the dtype);
 * diagram "Single-Pass mHC" (the hidden state is normalised) and "Cast to
 * MXFP8".
 *   y_norm[t][e] = dtype( x[t][e] / sqrt(mean_e x[t][e]^2 + norm_eps) * gain[e] )
 * and, for each group of 32 channels of a row of y_norm, with a = max |y_norm|
 * over the group:
 *   k = ceil(log2(max(a, 1e-4) / 448)),  scale[t][g] = k + 127 (UE8M0 byte),
 *   q[t][32g + i] = E4M3( clamp(y_norm[t][32g + i] / 2^k, -448, 448) )
 * (nearest E4M3 code, ties to even; sign kept).
 *   x [n][d] dtype, gain [d] fp32 in; y_norm [n][d] dtype, q [n][d] uint8,
 *   scale [n][d/32] uint8 out. y_norm may be NULL (the normalised row is then
 *   only cast); q and scale are both NULL (no cast) or both given; at least one
 *   output is required (HC_ERR_ARG otherwise). y_norm == x is allowed.
 *   d % 8 == 0, and d % 32 == 0 when casting (HC_ERR_UNSUPPORTED otherwise);
 *   q needs 8-byte alignment, scale any alignment; n < 2^31.
 */
int hc_rmsnorm_mxfp8(const void* x, int dtype, const float* gain, int64_t n, int64_t d,
                     float norm_eps, void* y_norm, uint8_t* q, uint8_t* scale, void* stream);

/*
 * One sublayer boundary of the single-pass design -- atlas "Block",
 * Block.forward; diagram "Single-Pass mHC".
 * If f_prev != NULL the previous sublayer's output is first written back:
 *   streams = hc_post(f_prev, residual, post_prev, comb_prev)  -> streams_out
 * otherwise streams = residual (streams_out, post_prev, comb_prev unused).
 * Then, from the (rounded) streams:
 *   mixes -> (pre, post, comb) as hc_mixes + hc_split_sinkhorn  (coefficients
 *            that THIS sublayer's hc_post and the NEXT collapse will use),
 *   y = hc_pre(streams, pre_mix), with pre_mix the collapse weights the
 *       previous sublayer produced (skipped when y == NULL).
 * mixes may be NULL (not stored). streams_out == residual is allowed.
 *   residual [n][hc][d], f_prev [n][d] dtype; post_prev [n][hc], comb_prev
 *   [n][hc][hc], pre_mix [n][hc], hc_fn [M][hc*d], hc_scale [3], hc_base [M]
 *   fp32 in; streams_out [n][hc][d], y [n][d] dtype out; pre, post [n][hc],
 *   comb [n][hc][hc], mixes [n][M] fp32 out.
 */
int hc_fused_step(const void* residual, const void* f_prev, const float* post_prev,
                  const float* comb_prev, const float* pre_mix, const float* hc_fn,
                  const float* hc_scale, const float* hc_base, int64_t n, int hc, int64_t d,
                  int dtype, float norm_eps, int sinkhorn_iters, float eps, void* streams_out,
                  void* y, float* pre, float* post, float* comb, float* mixes,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * hc_fused_step without a workspace argument, for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, validation, kernels and
 * results as hc_fused_step; its scratch (the per-slice partial rows) is a static
 * device array of HC_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends, looked up on a device's first call. The call
 * allocates nothing and never synchronises.
 *   - Sizes whose hc_workspace_size(n, hc, d) exceeds HC_NOALLOC_SCRATCH_BYTES are
 *     rejected with HC_ERR_SCRATCH before anything is enqueued (at d = 5120: up to
 *     262,144 tokens with four streams, 2,438 with eight).
 *   - All calls on one GPU share that GPU's scratch. Calls ordered on one stream
 *     are safe; calls that may overlap on one GPU (other streams without an
 *     ordering between them, other threads) race and must not be issued.
 *   - Nothing in the scratch has to start at zero: every partial row is written
 *     before it is read, so a previous call's contents do not matter.
 *   - HC_ERR_HIP also reports a failed lookup of the scratch's device address.
 */
int hc_fused_step_noalloc(const void* residual, const void* f_prev, const float* post_prev,
                          const float* comb_prev, const float* pre_mix, const float* hc_fn,
                          const float* hc_scale, const float* hc_base, int64_t n, int hc,
                          int64_t d, int dtype, float norm_eps, int sinkhorn_iters, float eps,
                          void* streams_out, void* y, float* pre, float* post, float* comb,
                          float* mixes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HC_H */
