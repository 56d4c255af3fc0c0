// hc_kernels.hip -- gfx950 kernels of the hyper-connection residual mix.
//
// Sources (page titles and sections):
//   atlas "Block", code section: Block.hc_mixes, Block.hc_pre, Block.hc_post,
//       Block.forward.
//   atlas "Stream combination", summary and code section (split + Sinkhorn).
//   diagram "DeepSeek-V4.1-Flash", blocks "Mixing Coefficients", "First Sinkhorn
//       Round", "Sinkhorn Round", "Single-Pass mHC".
//
// Kernels:
//   split_kernel        one lane per token: sigmoid split + Sinkhorn in registers.
//   pre_kernel          collapse, one lane per (token, 8 channels), 128-bit loads.
//   post_kernel         expand + combine, one lane per (token, 8 channels).
//   pass_kernel         one sweep over a tile of 64 tokens x a channel slice:
//                       optional expand (previous sublayer's post/comb), optional
//                       collapse, and the partial 24-wide projection + sum of
//                       squares of the (rounded) streams, written to a workspace.
//   finalize_kernel     one lane per token: reduce the slice partials in a fixed
//                       order, scale by the RMS statistic, and (optionally) split.
//
// All arithmetic is fp32. bf16 values are rounded to nearest-even
// (v_cvt_pk_bf16_f32). Buffer offsets are 64-bit throughout.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hc_internal.h"

namespace hc {
namespace {

typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kHC = 4;          // streams
constexpr int kMix = 24;        // (2 + hc) * hc mix numbers
constexpr int kPart = 32;       // floats per (split, token) partial row: 24 dots, sumsq, pad
constexpr int kWaves = 4;       // waves per pass workgroup
constexpr int kTokWave = 16;    // tokens per wave (one MFMA row tile)
constexpr int kTokWG = kWaves * kTokWave;
constexpr int kChunk = 32;      // channels per sweep step (4 lane groups x 8)

// ---------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t v = __builtin_convertvector((float2_t){a, b}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Eight consecutive elements of a row: load/store as fp32 values, plus the raw
// packed bf16 words (the MFMA operand) when the element type is bf16.
template <bool kBf16>
struct Vec8 {
    float v[8];
    uint4 raw;  // bf16 only

    __device__ __forceinline__ void load(const void* base, int64_t idx) {
        if constexpr (kBf16) {
            raw = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
            unpack();
        } else {
            const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
            float4 a = p[0], b = p[1];
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        }
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
        raw = make_uint4(0, 0, 0, 0);
    }
    __device__ __forceinline__ void unpack() {
        v[0] = bf16_lo(raw.x); v[1] = bf16_hi(raw.x);
        v[2] = bf16_lo(raw.y); v[3] = bf16_hi(raw.y);
        v[4] = bf16_lo(raw.z); v[5] = bf16_hi(raw.z);
        v[6] = bf16_lo(raw.w); v[7] = bf16_hi(raw.w);
    }
    // Round the fp32 values to the element type in place (bf16: RNE, and keep
    // the packed words); afterwards v[] holds exactly the stored values.
    __device__ __forceinline__ void round() {
        if constexpr (kBf16) {
            raw.x = pack_bf16x2(v[0], v[1]);
            raw.y = pack_bf16x2(v[2], v[3]);
            raw.z = pack_bf16x2(v[4], v[5]);
            raw.w = pack_bf16x2(v[6], v[7]);
            unpack();
        }
    }
    // Store (values must already be rounded for bf16).
    __device__ __forceinline__ void store(void* base, int64_t idx) const {
        if constexpr (kBf16) {
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx) = raw;
        } else {
            float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + idx);
            p[0] = make_float4(v[0], v[1], v[2], v[3]);
            p[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
};

// ------------------------------------------------------------- split/Sinkhorn
__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + __expf(-z)); }

// One token's split. m: its 24 mixes. scale/base: the sublayer's parameters
// (wave-uniform addresses: scalar loads). Normalisations multiply by a
// reciprocal of (sum + eps) computed once per row or column.
__device__ __forceinline__ void split_sinkhorn(const float (&m)[kMix], const float* __restrict__ scale,
                                               const float* __restrict__ base, int iters, float eps,
                                               float (&pre)[kHC], float (&post)[kHC],
                                               float (&C)[kHC * kHC]) {
    const float s0 = scale[0], s1 = scale[1], s2 = scale[2];
#pragma unroll
    for (int j = 0; j < kHC; ++j) {
        pre[j] = sigmoid(m[j] * s0 + base[j]) + eps;
        post[j] = 2.0f * sigmoid(m[kHC + j] * s1 + base[kHC + j]);
    }
#pragma unroll
    for (int i = 0; i < kHC * kHC; ++i) C[i] = m[2 * kHC + i] * s2 + base[2 * kHC + i];
    // first round: row softmax (max subtracted), + eps, column normalisation
#pragma unroll
    for (int j = 0; j < kHC; ++j) {
        float mx = fmaxf(fmaxf(C[4 * j], C[4 * j + 1]), fmaxf(C[4 * j + 2], C[4 * j + 3]));
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            C[4 * j + k] = __expf(C[4 * j + k] - mx);
            s += C[4 * j + k];
        }
        const float inv = __builtin_amdgcn_rcpf(s);
#pragma unroll
        for (int k = 0; k < kHC; ++k) C[4 * j + k] = C[4 * j + k] * inv + eps;
    }
    auto cols = [&]() {
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            const float inv = __builtin_amdgcn_rcpf(C[k] + C[4 + k] + C[8 + k] + C[12 + k] + eps);
#pragma unroll
            for (int j = 0; j < kHC; ++j) C[4 * j + k] *= inv;
        }
    };
    auto rows = [&]() {
#pragma unroll
        for (int j = 0; j < kHC; ++j) {
            const float inv =
                __builtin_amdgcn_rcpf(C[4 * j] + C[4 * j + 1] + C[4 * j + 2] + C[4 * j + 3] + eps);
#pragma unroll
            for (int k = 0; k < kHC; ++k) C[4 * j + k] *= inv;
        }
    };
    cols();
    for (int it = 1; it < iters; ++it) {
        rows();
        cols();
    }
}

__device__ __forceinline__ void store_coeffs(int64_t t, const float (&pre)[kHC], const float (&post)[kHC],
                                             const float (&C)[kHC * kHC], float* __restrict__ pre_out,
                                             float* __restrict__ post_out, float* __restrict__ comb_out) {
    reinterpret_cast<float4*>(pre_out)[t] = make_float4(pre[0], pre[1], pre[2], pre[3]);
    reinterpret_cast<float4*>(post_out)[t] = make_float4(post[0], post[1], post[2], post[3]);
    float4* cb = reinterpret_cast<float4*>(comb_out) + t * 4;
#pragma unroll
    for (int j = 0; j < kHC; ++j) cb[j] = make_float4(C[4 * j], C[4 * j + 1], C[4 * j + 2], C[4 * j + 3]);
}

constexpr int kSplitBlock = 256;

// One lane per token. The block's [256][24] logits are staged through LDS with
// 128-bit coalesced loads (row stride padded to 25 floats: no bank conflicts).
__global__ __launch_bounds__(kSplitBlock) void split_kernel(
    const float* __restrict__ mixes, const float* __restrict__ scale, const float* __restrict__ base,
    int64_t n, int iters, float eps, float* __restrict__ pre, float* __restrict__ post,
    float* __restrict__ comb) {
    __shared__ float tile[kSplitBlock * (kMix + 1)];
    const int64_t r0 = (int64_t)blockIdx.x * kSplitBlock;
    const int rows = (int)min<int64_t>(kSplitBlock, n - r0);
    const float4* src = reinterpret_cast<const float4*>(mixes + r0 * kMix);
    for (int q = threadIdx.x; q < rows * (kMix / 4); q += kSplitBlock) {
        const float4 v = src[q];
        const int e = q * 4, r = e / kMix, c = e - r * kMix;
        float* dst = tile + r * (kMix + 1) + c;
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
    __syncthreads();
    if ((int)threadIdx.x >= rows) return;
    float m[kMix];
#pragma unroll
    for (int i = 0; i < kMix; ++i) m[i] = tile[threadIdx.x * (kMix + 1) + i];
    float p[kHC], q[kHC], C[kHC * kHC];
    split_sinkhorn(m, scale, base, iters, eps, p, q, C);
    store_coeffs(r0 + threadIdx.x, p, q, C, pre, post, comb);
}

// ------------------------------------------------------------------ collapse
constexpr int kEwBlock = 256;

template <bool kBf16>
__global__ __launch_bounds__(kEwBlock) void pre_kernel(const void* __restrict__ x,
                                                       const float* __restrict__ pre_mix, int64_t n,
                                                       int64_t d, void* __restrict__ y) {
    const int64_t per_tok = d >> 3;
    const int64_t gid = (int64_t)blockIdx.x * kEwBlock + threadIdx.x;
    if (gid >= n * per_tok) return;
    const int64_t t = gid / per_tok;
    const int64_t e = (gid - t * per_tok) << 3;
    const float4 pm = reinterpret_cast<const float4*>(pre_mix)[t];
    const float w[kHC] = {pm.x, pm.y, pm.z, pm.w};
    Vec8<kBf16> out;
#pragma unroll
    for (int c = 0; c < 8; ++c) out.v[c] = 0.f;
#pragma unroll
    for (int j = 0; j < kHC; ++j) {
        Vec8<kBf16> xv;
        xv.load(x, (t * kHC + j) * d + e);
#pragma unroll
        for (int c = 0; c < 8; ++c) out.v[c] = fmaf(w[j], xv.v[c], out.v[c]);
    }
    out.round();
    out.store(y, t * d + e);
}

// ------------------------------------------------------------- expand/combine
template <bool kBf16>
__device__ __forceinline__ void expand8(const Vec8<kBf16>& f, const Vec8<kBf16> (&res)[kHC],
                                        const float (&post)[kHC], const float (&comb)[kHC * kHC],
                                        Vec8<kBf16> (&out)[kHC]) {
#pragma unroll
    for (int k = 0; k < kHC; ++k) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float a = post[k] * f.v[c];
#pragma unroll
            for (int j = 0; j < kHC; ++j) a = fmaf(comb[4 * j + k], res[j].v[c], a);
            out[k].v[c] = a;
        }
        out[k].round();
    }
}

template <bool kBf16>
__global__ __launch_bounds__(kEwBlock) void post_kernel(const void* __restrict__ f, const void* res,
                                                        const float* __restrict__ post,
                                                        const float* __restrict__ comb, int64_t n,
                                                        int64_t d, void* out) {
    const int64_t per_tok = d >> 3;
    const int64_t gid = (int64_t)blockIdx.x * kEwBlock + threadIdx.x;
    if (gid >= n * per_tok) return;
    const int64_t t = gid / per_tok;
    const int64_t e = (gid - t * per_tok) << 3;
    const float4 pv = reinterpret_cast<const float4*>(post)[t];
    const float pk[kHC] = {pv.x, pv.y, pv.z, pv.w};
    float cm[kHC * kHC];
#pragma unroll
    for (int j = 0; j < kHC; ++j) {
        const float4 c = reinterpret_cast<const float4*>(comb)[t * 4 + j];
        cm[4 * j] = c.x; cm[4 * j + 1] = c.y; cm[4 * j + 2] = c.z; cm[4 * j + 3] = c.w;
    }
    Vec8<kBf16> fv, rv[kHC], ov[kHC];
    fv.load(f, t * d + e);
#pragma unroll
    for (int j = 0; j < kHC; ++j) rv[j].load(res, (t * kHC + j) * d + e);
    expand8<kBf16>(fv, rv, pk, cm, ov);
#pragma unroll
    for (int k = 0; k < kHC; ++k) ov[k].store(out, (t * kHC + k) * d + e);
}

// ---------------------------------------------------------------- stream pass
// Workgroup = 4 waves x 16 tokens. Lane (r = lane % 16, g = lane / 16) of wave w
// owns token tile*64 + w*16 + r and, at sweep step ci, channels ci*32 + g*8 ..+8
// of all 4 streams. The step's slice of hc_fn (24 rows x 4 streams x 32 channels)
// is staged in LDS once per workgroup and shared by its 4 waves.
//
// Projection engines:
//   VALU  fp32 LDS copy of the slice; each lane accumulates 24 dot products
//         over its 32 values, then the 4 lane groups are summed with shuffles.
//   MFMA  (bf16 streams) the bf16 stream values are exact MFMA A operands; the
//         fp32 weights are split into three bf16 terms (hi + mid + lo, ~24
//         significant bits) stored in the B-operand layout of
//         v_mfma_f32_16x16x32_bf16; 24 mixes use two 16-wide column tiles
//         (rows 24..31 zero). Each term accumulates into the same fp32
//         accumulator.
struct PassArgs {
    const void* res;
    const void* f;
    const float* post_prev;
    const float* comb_prev;
    const float* pre_mix;
    const float* hc_fn;
    void* streams_out;
    void* y;
    float* part;
    int64_t n;
    int64_t d;
    int nchunks;
    int chunks_per_split;
};

constexpr int kPassBlock = kWaves * 64;
constexpr int kMfmaStage = 3 * 2 * kHC * 64;   // uint4 per LDS buffer: term x ntile x stream x lane
constexpr int kValuStage = kMix * kHC * kChunk; // floats per LDS buffer

template <bool kMfma>
struct PassLds;
template <>
struct PassLds<true> {
    uint4 b[2][kMfmaStage];
};
template <>
struct PassLds<false> {
    float w[2][kValuStage];
};

// Stage hc_fn[i][j*d + ci*32 + 0..31] for i < 24, j < 4 into LDS buffer `buf`.
template <bool kMfma>
__device__ __forceinline__ void stage_weights(PassLds<kMfma>& lds, int buf, const float* __restrict__ W,
                                              int64_t d, int ci) {
    const int64_t D = d * kHC;
#pragma unroll
    for (int q = 0; q < (kMix * kHC * kChunk / 4) / kPassBlock; ++q) {
        const int idx = threadIdx.x + q * kPassBlock;   // 0 .. 767
        const int i = idx >> 5;                         // mix row
        const int j = (idx >> 3) & 3;                   // stream
        const int c4 = idx & 7;                         // float4 within the 32 channels
        const int64_t e = (int64_t)ci * kChunk + c4 * 4;
        float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e < d) w = *reinterpret_cast<const float4*>(W + i * D + j * d + e);
        if constexpr (kMfma) {
            const float wv[4] = {w.x, w.y, w.z, w.w};
            uint32_t hi[2], mid[2], lo[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float a = wv[2 * h], b = wv[2 * h + 1];
                hi[h] = pack_bf16x2(a, b);
                const float ra = a - bf16_lo(hi[h]), rb = b - bf16_hi(hi[h]);
                mid[h] = pack_bf16x2(ra, rb);
                const float sa = ra - bf16_lo(mid[h]), sb = rb - bf16_hi(mid[h]);
                lo[h] = pack_bf16x2(sa, sb);
            }
            const int nt = i >> 4, col = i & 15;
            const int lane = (c4 >> 1) * 16 + col;
            const int half = c4 & 1;
            uint2* base = reinterpret_cast<uint2*>(lds.b[buf]);
            base[(((0 * 2 + nt) * kHC + j) * 64 + lane) * 2 + half] = make_uint2(hi[0], hi[1]);
            base[(((1 * 2 + nt) * kHC + j) * 64 + lane) * 2 + half] = make_uint2(mid[0], mid[1]);
            base[(((2 * 2 + nt) * kHC + j) * 64 + lane) * 2 + half] = make_uint2(lo[0], lo[1]);
        } else {
            reinterpret_cast<float4*>(lds.w[buf])[idx] = w;  // layout [i][j][32]
        }
    }
}

template <bool kBf16, bool kPost, bool kPre, bool kMfma>
__global__ __launch_bounds__(kPassBlock) void pass_kernel(PassArgs a) {
    static_assert(!kMfma || kBf16, "the MFMA engine needs bf16 stream values");
    __shared__ PassLds<kMfma> lds;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int64_t n = a.n, d = a.d;
    const int64_t t = (int64_t)blockIdx.x * kTokWG + wave * kTokWave + r;
    const bool tok_ok = t < n;
    const int split = blockIdx.y;
    const int c_begin = split * a.chunks_per_split;
    const int c_end = min(a.nchunks, c_begin + a.chunks_per_split);

    if constexpr (kMfma) {
        // the B rows 24..31 (tile 1, columns 8..15) stay zero for the whole sweep
        for (int z = threadIdx.x; z < 2 * 3 * kHC * 4 * 8; z += kPassBlock) {
            const int col = 8 + (z & 7), gg = (z >> 3) & 3, j = (z >> 5) & 3, term = (z >> 7) % 3,
                      buf = z / (3 * kHC * 4 * 8);
            lds.b[buf][((term * 2 + 1) * kHC + j) * 64 + gg * 16 + col] = make_uint4(0, 0, 0, 0);
        }
    }

    float pk[kHC] = {0.f, 0.f, 0.f, 0.f}, cm[kHC * kHC], pim[kHC] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kHC * kHC; ++i) cm[i] = 0.f;
    if (tok_ok) {
        if constexpr (kPost) {
            const float4 pv = reinterpret_cast<const float4*>(a.post_prev)[t];
            pk[0] = pv.x; pk[1] = pv.y; pk[2] = pv.z; pk[3] = pv.w;
#pragma unroll
            for (int j = 0; j < kHC; ++j) {
                const float4 c = reinterpret_cast<const float4*>(a.comb_prev)[t * 4 + j];
                cm[4 * j] = c.x; cm[4 * j + 1] = c.y; cm[4 * j + 2] = c.z; cm[4 * j + 3] = c.w;
            }
        }
        if constexpr (kPre) {
            const float4 pv = reinterpret_cast<const float4*>(a.pre_mix)[t];
            pim[0] = pv.x; pim[1] = pv.y; pim[2] = pv.z; pim[3] = pv.w;
        }
    }

    floatx4_t acc_m[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float acc_v[kMix];
#pragma unroll
    for (int i = 0; i < kMix; ++i) acc_v[i] = 0.f;
    float sumsq = 0.f;

    if (c_begin < c_end) stage_weights<kMfma>(lds, 0, a.hc_fn, d, c_begin);
    __syncthreads();

    for (int ci = c_begin; ci < c_end; ++ci) {
        const int buf = (ci - c_begin) & 1;
        if (ci + 1 < c_end) stage_weights<kMfma>(lds, buf ^ 1, a.hc_fn, d, ci + 1);

        const int64_t e = (int64_t)ci * kChunk + g * 8;
        const bool live = tok_ok && e < d;
        Vec8<kBf16> xs[kHC];
        if (live) {
#pragma unroll
            for (int j = 0; j < kHC; ++j) xs[j].load(a.res, (t * kHC + j) * d + e);
        } else {
#pragma unroll
            for (int j = 0; j < kHC; ++j) xs[j].zero();
        }
        if constexpr (kPost) {
            Vec8<kBf16> fv, x1[kHC];
            if (live) fv.load(a.f, t * d + e);
            else fv.zero();
            expand8<kBf16>(fv, xs, pk, cm, x1);
#pragma unroll
            for (int k = 0; k < kHC; ++k) {
                if (live) x1[k].store(a.streams_out, (t * kHC + k) * d + e);
                xs[k] = x1[k];
            }
        }
        if constexpr (kPre) {
            Vec8<kBf16> yv;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < kHC; ++j) s = fmaf(pim[j], xs[j].v[c], s);
                yv.v[c] = s;
            }
            yv.round();
            if (live) yv.store(a.y, t * d + e);
        }
#pragma unroll
        for (int j = 0; j < kHC; ++j)
#pragma unroll
            for (int c = 0; c < 8; ++c) sumsq = fmaf(xs[j].v[c], xs[j].v[c], sumsq);

        if constexpr (kMfma) {
            const uint4* B = lds.b[buf];
#pragma unroll
            for (int j = 0; j < kHC; ++j) {
                const bf16x8_t A = __builtin_bit_cast(bf16x8_t, xs[j].raw);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int term = 0; term < 3; ++term) {
                        const bf16x8_t Bv =
                            __builtin_bit_cast(bf16x8_t, B[((term * 2 + nt) * kHC + j) * 64 + lane]);
                        acc_m[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bv, acc_m[nt], 0, 0, 0);
                    }
            }
        } else {
            const float4* W = reinterpret_cast<const float4*>(lds.w[buf]);
#pragma unroll
            for (int i = 0; i < kMix; ++i) {
                float s = acc_v[i];
#pragma unroll
                for (int j = 0; j < kHC; ++j) {
                    const float4 w0 = W[((i * kHC + j) * kChunk + g * 8) / 4];
                    const float4 w1 = W[((i * kHC + j) * kChunk + g * 8) / 4 + 1];
                    s = fmaf(w0.x, xs[j].v[0], s); s = fmaf(w0.y, xs[j].v[1], s);
                    s = fmaf(w0.z, xs[j].v[2], s); s = fmaf(w0.w, xs[j].v[3], s);
                    s = fmaf(w1.x, xs[j].v[4], s); s = fmaf(w1.y, xs[j].v[5], s);
                    s = fmaf(w1.z, xs[j].v[6], s); s = fmaf(w1.w, xs[j].v[7], s);
                }
                acc_v[i] = s;
            }
        }
        __syncthreads();
    }

    // partial results of this (token tile, channel slice)
    float* part = a.part + (int64_t)split * n * kPart;
    sumsq += __shfl_xor(sumsq, 16);
    sumsq += __shfl_xor(sumsq, 32);
    if (g == 0 && tok_ok) part[t * kPart + kMix] = sumsq;
    if constexpr (kMfma) {
        // accumulator layout: lane holds rows 4*g .. 4*g+3 (tokens), column r (mix)
        const int64_t t0 = (int64_t)blockIdx.x * kTokWG + wave * kTokWave + 4 * g;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int mix = nt * 16 + r;
            if (mix < kMix) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    if (t0 + ii < n) part[(t0 + ii) * kPart + mix] = acc_m[nt][ii];
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kMix; ++i) {
            float s = acc_v[i];
            s += __shfl_xor(s, 16);
            s += __shfl_xor(s, 32);
            acc_v[i] = s;
        }
        if (g == 0 && tok_ok) {
            float4* dst = reinterpret_cast<float4*>(part + t * kPart);
#pragma unroll
            for (int q = 0; q < kMix / 4; ++q)
                dst[q] = make_float4(acc_v[4 * q], acc_v[4 * q + 1], acc_v[4 * q + 2], acc_v[4 * q + 3]);
        }
    }
}

// ------------------------------------------------------------------ finalize
template <bool kSplit>
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ part, int nsplit,
                                                       int64_t n, int64_t D, float norm_eps,
                                                       const float* __restrict__ scale,
                                                       const float* __restrict__ base, int iters,
                                                       float eps, float* __restrict__ mixes,
                                                       float* __restrict__ pre, float* __restrict__ post,
                                                       float* __restrict__ comb) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n) return;
    float acc[kMix + 1];
#pragma unroll
    for (int i = 0; i <= kMix; ++i) acc[i] = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const float* p = part + ((int64_t)s * n + t) * kPart;
        const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll
        for (int q = 0; q < kMix / 4; ++q) {
            const float4 v = p4[q];
            acc[4 * q] += v.x; acc[4 * q + 1] += v.y; acc[4 * q + 2] += v.z; acc[4 * q + 3] += v.w;
        }
        acc[kMix] += p[kMix];
    }
    const float rstd = 1.0f / sqrtf(acc[kMix] / (float)D + norm_eps);
    float m[kMix];
#pragma unroll
    for (int i = 0; i < kMix; ++i) m[i] = acc[i] * rstd;
    if (mixes) {
        float4* dst = reinterpret_cast<float4*>(mixes + t * kMix);
#pragma unroll
        for (int q = 0; q < kMix / 4; ++q) dst[q] = make_float4(m[4 * q], m[4 * q + 1], m[4 * q + 2], m[4 * q + 3]);
    }
    if constexpr (kSplit) {
        float p[kHC], q[kHC], C[kHC * kHC];
        split_sinkhorn(m, scale, base, iters, eps, p, q, C);
        store_coeffs(t, p, q, C, pre, post, comb);
    }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// ------------------------------------------------------------------- launchers
PassPlan plan_pass(int64_t n, int64_t d) {
    PassPlan p{};
    p.tiles = ceil_div(n, kTokWG);
    p.nchunks = (int)ceil_div(d, kChunk);
    const int64_t target_groups = 512;
    int64_t ns = ceil_div(target_groups, p.tiles > 0 ? p.tiles : 1);
    if (ns < 1) ns = 1;
    if (ns > p.nchunks) ns = p.nchunks;
    if (ns > 64) ns = 64;
    p.chunks_per_split = (int)ceil_div(p.nchunks, ns);
    p.nsplit = (int)ceil_div(p.nchunks, p.chunks_per_split);
    p.workspace_bytes = (size_t)p.nsplit * (size_t)n * kPart * sizeof(float);
    return p;
}

hipError_t launch_split(const float* mixes, const float* scale, const float* base, int64_t n, int iters,
                        float eps, float* pre, float* post, float* comb, hipStream_t stream) {
    hipLaunchKernelGGL(split_kernel, dim3((unsigned)ceil_div(n, kSplitBlock)), dim3(kSplitBlock), 0, stream,
                       mixes, scale, base, n, iters, eps, pre, post, comb);
    return hipGetLastError();
}

hipError_t launch_pre(const void* x, bool bf16, const float* pre_mix, int64_t n, int64_t d, void* y,
                      hipStream_t stream) {
    const dim3 grid((unsigned)ceil_div(n * (d / 8), kEwBlock));
    if (bf16)
        hipLaunchKernelGGL(pre_kernel<true>, grid, dim3(kEwBlock), 0, stream, x, pre_mix, n, d, y);
    else
        hipLaunchKernelGGL(pre_kernel<false>, grid, dim3(kEwBlock), 0, stream, x, pre_mix, n, d, y);
    return hipGetLastError();
}

hipError_t launch_post(const void* f, const void* res, bool bf16, const float* post, const float* comb,
                       int64_t n, int64_t d, void* out, hipStream_t stream) {
    const dim3 grid((unsigned)ceil_div(n * (d / 8), kEwBlock));
    if (bf16)
        hipLaunchKernelGGL(post_kernel<true>, grid, dim3(kEwBlock), 0, stream, f, res, post, comb, n, d, out);
    else
        hipLaunchKernelGGL(post_kernel<false>, grid, dim3(kEwBlock), 0, stream, f, res, post, comb, n, d, out);
    return hipGetLastError();
}

namespace {
template <bool kBf16, bool kPost, bool kPre, bool kMfma>
void launch_pass_t(const PassArgs& a, const PassPlan& p, hipStream_t stream) {
    hipLaunchKernelGGL((pass_kernel<kBf16, kPost, kPre, kMfma>), dim3((unsigned)p.tiles, (unsigned)p.nsplit),
                       dim3(kPassBlock), 0, stream, a);
}

template <bool kBf16, bool kMfma>
void launch_pass_flags(const PassArgs& a, const PassPlan& p, bool post, bool pre, hipStream_t stream) {
    if (post && pre) launch_pass_t<kBf16, true, true, kMfma>(a, p, stream);
    else if (post) launch_pass_t<kBf16, true, false, kMfma>(a, p, stream);
    else if (pre) launch_pass_t<kBf16, false, true, kMfma>(a, p, stream);
    else launch_pass_t<kBf16, false, false, kMfma>(a, p, stream);
}
}  // namespace

hipError_t launch_pass_and_finalize(const PassRequest& r, hipStream_t stream) {
    const PassPlan p = plan_pass(r.n, r.d);
    PassArgs a{};
    a.res = r.res;
    a.f = r.f_prev;
    a.post_prev = r.post_prev;
    a.comb_prev = r.comb_prev;
    a.pre_mix = r.pre_mix;
    a.hc_fn = r.hc_fn;
    a.streams_out = r.streams_out;
    a.y = r.y;
    a.part = static_cast<float*>(r.workspace);
    a.n = r.n;
    a.d = r.d;
    a.nchunks = p.nchunks;
    a.chunks_per_split = p.chunks_per_split;
    const bool post = r.f_prev != nullptr, pre = r.y != nullptr;
    // Projection engine: VALU for every stream dtype.
    if (r.bf16) launch_pass_flags<true, false>(a, p, post, pre, stream);
    else launch_pass_flags<false, false>(a, p, post, pre, stream);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 fgrid((unsigned)ceil_div(r.n, 256));
    if (r.split)
        hipLaunchKernelGGL(finalize_kernel<true>, fgrid, dim3(256), 0, stream, a.part, p.nsplit, r.n,
                           r.d * kHC, r.norm_eps, r.scale, r.base, r.iters, r.eps, r.mixes, r.pre, r.post,
                           r.comb);
    else
        hipLaunchKernelGGL(finalize_kernel<false>, fgrid, dim3(256), 0, stream, a.part, p.nsplit, r.n,
                           r.d * kHC, r.norm_eps, r.scale, r.base, r.iters, r.eps, r.mixes, r.pre, r.post,
                           r.comb);
    return hipGetLastError();
}

}  // namespace hc
