/*
 * hc_oracle.c -- plain, slow CPU oracle for the hyper-connection residual mix.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the reference against which the HIP
 * library is checked. Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it. It shares no code, header or table with the
 * HIP path and must never be linked into it.
 *
 * Sources (page titles; sections named, no line numbers):
 *   [Block]     atlas page "Block" (DeepSeek-V4.1, reindex-groups layer):
 *               code section, methods Block.hc_mixes, Block.hc_pre,
 *               Block.hc_post and Block.forward; parameter table.
 *   [Combine]   atlas page "Stream combination" (DeepSeek-V4.1 attention stream
 *               weights): summary paragraph, code section (the split/Sinkhorn
 *               kernel and its wrapper), released configuration.
 *   [Diagram]   "DeepSeek-V4.1-Flash" diagram page: blocks "Mixing
 *               Coefficients", "sigma", "x + eps_hc", "2 sigma",
 *               "First Sinkhorn Round", "Sinkhorn Round", "Cast",
 *               "Single-Pass mHC" (the hidden state is normalised after the
 *               collapse), "Cast to MXFP8".
 *   [Donor]     "DeepSeek-R1 donor reference" page: the RMSNorm passages
 *               ("Normalize by the root mean square", "Apply learned
 *               per-feature RMSNorm gains").
 *
 * Arithmetic: every sum and product is carried out in double precision
 * (fp64). A value is rounded exactly once, to the precision of the tensor the
 * pages materialise it in:
 *   mixes, pre, post, comb  -> fp32   ([Block] hc_mixes; [Combine] kernel outputs)
 *   collapsed input y       -> stream dtype ([Block] hc_pre casts back)
 *   new streams x'          -> dtype of the sublayer output ([Block] hc_post)
 * bf16 rounding is round-to-nearest, ties to even, applied to the fp64 value
 * ([Diagram] "Cast": the nearest representable number).
 *
 * Layouts (row-major, contiguous):
 *   x, residual, out : [n][hc][d]       stream index j, channel e
 *   f, y             : [n][d]
 *   hc_fn            : [(2+hc)*hc][hc*d] flattened input index c = j*d + e
 *   mixes            : [n][(2+hc)*hc]    pre logits | post logits | comb logits
 *   pre, post        : [n][hc]
 *   comb             : [n][hc][hc]       comb[j][k]: j = source (old) stream,
 *                                        k = destination (new) stream
 * dtype codes: 0 = fp32, 1 = bf16 (bf16 data is passed as raw 16-bit words).
 *
 * Return value of every function: 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* bf16 -> double: the bf16 word is the upper half of an fp32 word, so the
 * value widens exactly ([Diagram] "Cast" BF16 -> FP32 changes no value). */
static double bf16_bits_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* double -> bf16, round to nearest, ties to even, straight from fp64 (no
 * intermediate fp32 rounding). bf16 keeps 8 significant bits and the fp32
 * exponent range (normal down to 2^-126, subnormal step 2^-133). */
static uint16_t double_to_bf16_bits(double v)
{
    if (isnan(v))
        return 0x7fc0;
    double a = fabs(v);
    double q;
    if (a == 0.0) {
        q = 0.0;
    } else if (a < ldexp(1.0, -126)) {
        /* subnormal range: multiples of 2^-133 */
        q = ldexp(nearbyint(ldexp(a, 133)), -133);
    } else {
        int e;
        double m = frexp(a, &e);            /* a = m * 2^e, m in [0.5, 1) */
        double s = nearbyint(ldexp(m, 8));  /* 8 significant bits, ties-to-even */
        q = ldexp(s, e - 8);
    }
    /* exact below 2^128 (q has <= 8 significant bits); 2^128 and beyond is
     * infinity, tested before the conversion (a double out of the float range
     * has no defined conversion) */
    float qf = q >= ldexp(1.0, 128) ? INFINITY : (float)q;
    if (v < 0)
        qf = -qf;
    uint32_t u;
    memcpy(&u, &qf, sizeof u);
    return (uint16_t)(u >> 16);
}

static double load_elem(const void* p, int dtype, int64_t i)
{
    if (dtype == ORACLE_BF16)
        return bf16_bits_to_double(((const uint16_t*)p)[i]);
    return (double)((const float*)p)[i];
}

static void store_elem(void* p, int dtype, int64_t i, double v)
{
    if (dtype == ORACLE_BF16)
        ((uint16_t*)p)[i] = double_to_bf16_bits(v);
    else
        ((float*)p)[i] = (float)v;  /* C conversion rounds to nearest-even */
}

static int bad_dtype(int dtype) { return dtype != ORACLE_F32 && dtype != ORACLE_BF16; }

/* Exposed for the rounding pins in the test suite. */
uint16_t oracle_round_bf16(double v) { return double_to_bf16_bits(v); }

/*
 * a1-a3: mix projection ([Block] hc_mixes; [Diagram] "Mixing Coefficients").
 * For token t the hc streams are flattened into one vector of length D = hc*d
 * and widened to real numbers. One RMS statistic is taken over all D entries,
 * r = 1/sqrt(mean(x^2) + norm_eps), and each of the (2+hc)*hc rows of hc_fn is
 * dotted with the (unnormalised) vector; the dot product is then multiplied by
 * r. The released configuration sets norm_eps = 1e-20.
 */
int oracle_hc_mixes(const void* x, int dtype, int64_t n, int hc, int64_t d,
                    const float* hc_fn, double norm_eps, float* mixes)
{
    if (n < 0 || hc < 1 || d < 1 || bad_dtype(dtype))
        return -1;
    if (n == 0)
        return 0;
    if (!x || !hc_fn || !mixes)
        return -1;
    const int64_t D = (int64_t)hc * d;
    const int M = (2 + hc) * hc;
    double* row = (double*)malloc((size_t)D * sizeof(double));
    if (!row)
        return -1;
    for (int64_t t = 0; t < n; ++t) {
        double sumsq = 0.0;
        for (int64_t c = 0; c < D; ++c) {
            row[c] = load_elem(x, dtype, t * D + c);
            sumsq += row[c] * row[c];
        }
        double r = 1.0 / sqrt(sumsq / (double)D + norm_eps);
        for (int i = 0; i < M; ++i) {
            const float* w = hc_fn + (int64_t)i * D;
            double dot = 0.0;
            for (int64_t c = 0; c < D; ++c)
                dot += (double)w[c] * row[c];
            mixes[t * M + i] = (float)(dot * r);
        }
    }
    free(row);
    return 0;
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* Divide every row of the hc x hc matrix by (its sum + eps). */
static void normalise_rows(double* C, int hc, double eps)
{
    for (int j = 0; j < hc; ++j) {
        double s = 0.0;
        for (int k = 0; k < hc; ++k)
            s += C[j * hc + k];
        for (int k = 0; k < hc; ++k)
            C[j * hc + k] /= (s + eps);
    }
}

/* Divide every column of the hc x hc matrix by (its sum + eps). */
static void normalise_cols(double* C, int hc, double eps)
{
    for (int k = 0; k < hc; ++k) {
        double s = 0.0;
        for (int j = 0; j < hc; ++j)
            s += C[j * hc + k];
        for (int j = 0; j < hc; ++j)
            C[j * hc + k] /= (s + eps);
    }
}

/*
 * a4: split and Sinkhorn ([Combine] summary and code section; [Diagram]
 * "sigma", "x + eps_hc", "2 sigma", "First Sinkhorn Round", "Sinkhorn Round").
 * With s = hc_scale[0..2], b = hc_base, m = the token's mixes:
 *   pre[j]  = sigmoid(s0*m[j] + b[j]) + eps
 *   post[j] = 2*sigmoid(s1*m[hc+j] + b[hc+j])
 *   L[j][k] = s2*m[2hc + j*hc + k] + b[2hc + j*hc + k]
 * First round: softmax along each row (max subtracted before exp), eps added
 * to every entry, then every column divided by (column sum + eps).
 * Each later round (sinkhorn_iters - 1 of them): every row divided by
 * (row sum + eps), then every column divided by (column sum + eps).
 */
int oracle_hc_split_sinkhorn(const float* mixes, const float* hc_scale, const float* hc_base,
                             int64_t n, int hc, int sinkhorn_iters, double eps,
                             float* pre, float* post, float* comb)
{
    if (n < 0 || hc < 1 || sinkhorn_iters < 1 || !(eps >= 0.0))
        return -1;
    if (n == 0)
        return 0;
    if (!mixes || !hc_scale || !hc_base || !pre || !post || !comb)
        return -1;
    const int M = (2 + hc) * hc;
    double* C = (double*)malloc((size_t)hc * hc * sizeof(double));
    if (!C)
        return -1;
    const double s0 = hc_scale[0], s1 = hc_scale[1], s2 = hc_scale[2];
    for (int64_t t = 0; t < n; ++t) {
        const float* m = mixes + t * M;
        for (int j = 0; j < hc; ++j)
            pre[t * hc + j] = (float)(sigmoid(s0 * m[j] + hc_base[j]) + eps);
        for (int j = 0; j < hc; ++j)
            post[t * hc + j] = (float)(2.0 * sigmoid(s1 * m[hc + j] + hc_base[hc + j]));
        for (int j = 0; j < hc; ++j)
            for (int k = 0; k < hc; ++k) {
                int i = 2 * hc + j * hc + k;
                C[j * hc + k] = s2 * m[i] + hc_base[i];
            }
        /* first round: row softmax, + eps, column normalisation */
        for (int j = 0; j < hc; ++j) {
            double mx = C[j * hc];
            for (int k = 1; k < hc; ++k)
                if (C[j * hc + k] > mx)
                    mx = C[j * hc + k];
            double s = 0.0;
            for (int k = 0; k < hc; ++k) {
                C[j * hc + k] = exp(C[j * hc + k] - mx);
                s += C[j * hc + k];
            }
            for (int k = 0; k < hc; ++k)
                C[j * hc + k] = C[j * hc + k] / s + eps;
        }
        normalise_cols(C, hc, eps);
        /* the remaining rounds */
        for (int it = 1; it < sinkhorn_iters; ++it) {
            normalise_rows(C, hc, eps);
            normalise_cols(C, hc, eps);
        }
        for (int i = 0; i < hc * hc; ++i)
            comb[t * hc * hc + i] = (float)C[i];
    }
    free(C);
    return 0;
}

/*
 * a5: collapse ([Block] hc_pre). y[t][e] = sum_j pre_mix[t][j] * x[t][j][e],
 * summed over the hc streams, rounded once to the stream dtype.
 */
int oracle_hc_pre(const void* x, int dtype, const float* pre_mix, int64_t n, int hc, int64_t d,
                  void* y)
{
    if (n < 0 || hc < 1 || d < 1 || bad_dtype(dtype))
        return -1;
    if (n == 0)
        return 0;
    if (!x || !pre_mix || !y)
        return -1;
    for (int64_t t = 0; t < n; ++t)
        for (int64_t e = 0; e < d; ++e) {
            double acc = 0.0;
            for (int j = 0; j < hc; ++j)
                acc += (double)pre_mix[t * hc + j] * load_elem(x, dtype, (t * hc + j) * d + e);
            store_elem(y, dtype, t * d + e, acc);
        }
    return 0;
}

/*
 * a6: expand and combine ([Block] hc_post).
 * out[t][k][e] = post[t][k]*f[t][e] + sum_j comb[t][j][k]*residual[t][j][e]:
 * the sum runs over the FIRST index of comb (the source stream), so new stream
 * k takes the weights of column k. Rounded once to the dtype of f, which is
 * also the dtype of residual.
 */
int oracle_hc_post(const void* f, const void* residual, int dtype, const float* post,
                   const float* comb, int64_t n, int hc, int64_t d, void* out)
{
    if (n < 0 || hc < 1 || d < 1 || bad_dtype(dtype))
        return -1;
    if (n == 0)
        return 0;
    if (!f || !residual || !post || !comb || !out)
        return -1;
    for (int64_t t = 0; t < n; ++t)
        for (int k = 0; k < hc; ++k)
            for (int64_t e = 0; e < d; ++e) {
                double acc = (double)post[t * hc + k] * load_elem(f, dtype, t * d + e);
                for (int j = 0; j < hc; ++j)
                    acc += (double)comb[(t * hc + j) * hc + k] *
                           load_elem(residual, dtype, (t * hc + j) * d + e);
                store_elem(out, dtype, (t * hc + k) * d + e, acc);
            }
    return 0;
}


/*
 * Sublayer RMSNorm after the collapse ([Block] Block.forward applies attn_norm /
 * ffn_norm, RMSNorm(dim, norm_eps), to the collapsed input; [Donor] RMSNorm
 * passages; [Diagram] "Single-Pass mHC").
 * out[t][e] = x[t][e] / sqrt(mean_e x[t][e]^2 + eps) * gain[e], over the d
 * channels of the row, rounded once to the dtype of x (the gain multiplies the
 * scaled value, then the earlier dtype is restored).
 */
int oracle_rmsnorm(const void* x, int dtype, int64_t n, int64_t d, const float* gain, double eps,
                   void* out)
{
    if (n < 0 || d < 1 || bad_dtype(dtype) || !(eps >= 0.0))
        return -1;
    if (n == 0)
        return 0;
    if (!x || !gain || !out)
        return -1;
    for (int64_t t = 0; t < n; ++t) {
        double ss = 0.0;
        for (int64_t e = 0; e < d; ++e) {
            const double v = load_elem(x, dtype, t * d + e);
            ss += v * v;
        }
        const double r = 1.0 / sqrt(ss / (double)d + eps);
        for (int64_t e = 0; e < d; ++e)
            store_elem(out, dtype, t * d + e, load_elem(x, dtype, t * d + e) * r * (double)gain[e]);
    }
    return 0;
}

/* E4M3 (4 exponent bits, bias 7, 3 mantissa bits; largest finite 448, smallest
 * subnormal 2^-9) of a value with |v| <= 448, rounded to the nearest code, ties
 * to the even code; the sign is kept (a value that rounds to zero keeps it). */
static uint8_t e4m3_code(double v)
{
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const double a = fabs(v);
    if (a < ldexp(1.0, -6)) {                     /* subnormal codes: multiples of 2^-9 */
        const double q = nearbyint(ldexp(a, 9));   /* 0..8; 8 is the smallest normal */
        return sign | (uint8_t)q;
    }
    int e;
    const double m = frexp(a, &e);                 /* a = m * 2^e, m in [0.5, 1) */
    int exp = e - 1;                               /* a = (2m) * 2^exp, 2m in [1, 2) */
    double mant = nearbyint((2.0 * m - 1.0) * 8.0);   /* 3 fraction bits, ties to even */
    if (mant == 8.0) {
        mant = 0.0;
        exp += 1;
    }
    return sign | (uint8_t)(((exp + 7) << 3) | (int)mant);
}

/* ceil(log2(v)) for v > 0, exactly (frexp: v = m * 2^e, m in [0.5, 1)). */
static int ceil_log2(double v)
{
    int e;
    const double m = frexp(v, &e);
    return m == 0.5 ? e - 1 : e;
}

/*
 * MXFP8 cast ([Diagram] "Cast to MXFP8"): the channels of a row are cut into
 * groups of 32. Group g: a = max |x| over the group; its scale is the power of two
 * s = 2^ceil(log2(max(a, 1e-4) / 448)), stored as the UE8M0 byte log2(s) + 127;
 * each element is x / s, clamped to [-448, 448] and rounded to the nearest E4M3
 * code. d must be a multiple of 32. x / s is exact (s is a power of two), and
 * since s >= a / 448 the clamp never acts; it is kept as the page states it.
 */
int oracle_mxfp8(const void* x, int dtype, int64_t n, int64_t d, uint8_t* q, uint8_t* scale)
{
    if (n < 0 || d < 32 || d % 32 != 0 || bad_dtype(dtype))
        return -1;
    if (n == 0)
        return 0;
    if (!x || !q || !scale)
        return -1;
    for (int64_t t = 0; t < n; ++t)
        for (int64_t g = 0; g < d / 32; ++g) {
            double a = 0.0;
            for (int i = 0; i < 32; ++i) {
                const double v = fabs(load_elem(x, dtype, t * d + g * 32 + i));
                if (v > a)
                    a = v;
            }
            const int k = ceil_log2((a > 1e-4 ? a : 1e-4) / 448.0);
            scale[t * (d / 32) + g] = (uint8_t)(k + 127);
            for (int i = 0; i < 32; ++i) {
                double v = ldexp(load_elem(x, dtype, t * d + g * 32 + i), -k);
                if (v > 448.0)
                    v = 448.0;
                if (v < -448.0)
                    v = -448.0;
                q[t * d + g * 32 + i] = e4m3_code(v);
            }
        }
    return 0;
}
