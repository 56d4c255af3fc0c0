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
//   finalize_kernel     16 lanes per token: reduce the slice partials in a fixed
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
#ifndef HC_TILES
#define HC_TILES 1
#endif
#ifndef HC_TARGET_GROUPS
#define HC_TARGET_GROUPS 512
#endif
constexpr int kWaves = 4;           // waves per pass workgroup
constexpr int kTiles = HC_TILES;    // 16-token MFMA row tiles per wave
constexpr int kTokWave = 16 * kTiles;
constexpr int kTokWG = kWaves * kTokWave;
constexpr int kChunk = 32;      // channels per sweep step (4 lane groups x 8)

// ---------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t v = __builtin_convertvector((float2_t){a, b}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ------------------------------------------------------------- buffer access
// Raw buffer loads/stores (MUBUF): a wave-uniform 128-bit resource (base, byte
// range) plus a per-lane 32-bit offset and a uniform scalar offset. A lane whose
// offset is kOffMasked lies outside the range: its load returns zeros and its
// store is dropped. The range is capped below 2^31 so that holds for any tensor.
// The range check covers the per-lane offset only (the scalar offset is excluded),
// so every lane that must not touch memory gets kOffMasked explicitly.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr uint32_t kOffMasked = 0x80000000u;
constexpr int kRawBufferFlags = 0x00020000;   // 32-bit data format, raw addressing

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int64_t b = bytes < 0 ? 0 : (bytes > 0x7ffffff0 ? 0x7ffffff0 : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)b, kRawBufferFlags);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 buf_load16f(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
__device__ __forceinline__ void buf_store16(uint4 v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, (int)voff, (int)soff, 0);
}

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
// Projection engines (A = 16 tokens x k, B = k x 16 mixes, fp32 accumulators;
// the 24 mixes use two 16-wide column tiles whose columns 24..31 are zero):
//   bf16 streams: v_mfma_f32_16x16x32_bf16. The bf16 stream values are exact A
//         operands; the fp32 weights are split into three bf16 terms (hi + mid +
//         lo, ~24 significant bits), each accumulated into the same accumulator.
//   fp32 streams: v_mfma_f32_16x16x4f32 with the fp32 values and weights as they
//         are; k runs over the 4 lane groups, one MFMA per (stream, channel).
//
// Pipelining: while step ci is computed, the stream values of step ci+1 are
// already loaded into registers and its weights fetched; the weights are split
// into the other LDS buffer after step ci's MFMAs, then one barrier per step.
//
// Grid: one dimension, workgroup L -> (tile = L / nsplit, slice = L % nsplit).
// Workgroups are dealt to the 8 XCDs round-robin, so with nsplit a multiple of 8
// every XCD works on a fixed set of channel slices and its L2 holds only that
// part of hc_fn.
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
    int nsplit;
};

constexpr int kPassBlock = kWaves * 64;
constexpr int kBf16Stage = 3 * 2 * kHC * 64;   // uint4 per LDS buffer: term x ntile x stream x lane
constexpr int kF32Row = kHC * kChunk + 4;      // floats per mix row of the fp32 stage (padded)
constexpr int kF32Stage = 32 * kF32Row;        // floats per LDS buffer: 32 mix rows (24..31 zero)
constexpr int kStageLoads = (kMix * kHC * kChunk / 4) / kPassBlock;  // float4 per thread per step

// B-fragment slot (16 B) of (term, ntile, stream j, lane) in a bf16 weight stage,
// XOR-swizzled within groups of 8 so that the split's 8-byte writes spread over
// all banks while the MFMA's lane-ordered 16-byte reads stay conflict-free.
// Columns 8..15 of a slot group stay in 8..15 (padding maps onto padding).
__device__ __forceinline__ int b_slot(int term, int nt, int j, int lane) {
    const int slot = ((term * 2 + nt) * 4 + j) * 64 + lane;
    return slot ^ (((lane >> 4) + 4 * (j & 1)) & 7);
}

template <bool kBf16>
struct PassLds;
template <>
struct PassLds<true> {
    uint4 b[2][kBf16Stage];
};
template <>
struct PassLds<false> {
    float w[2][kF32Stage];
};

__device__ __forceinline__ uint4* lds_b(PassLds<true>& l, int buf) { return l.b[buf]; }
__device__ __forceinline__ uint4* lds_b(PassLds<false>&, int) { return nullptr; }
__device__ __forceinline__ float* lds_w(PassLds<false>& l, int buf) { return l.w[buf]; }
__device__ __forceinline__ float* lds_w(PassLds<true>&, int) { return nullptr; }

// Thread's share of hc_fn[i][j*d + ci*32 + 0..31] (i < 24, j < 4): kStageLoads
// float4 values; entry q covers idx = threadIdx.x + q*256 -> i = idx/32,
// j = (idx/8)%4, 4 channels at (idx%8)*4. Channels past d read as zero: the load
// itself always targets an in-bounds address (clamped) and the value is masked,
// so no load sits behind a branch.
__device__ __forceinline__ void fetch_weights(float4 (&w)[kStageLoads], const float* __restrict__ W,
                                              int64_t d, int ci) {
    const int64_t D = d * kHC;
#pragma unroll
    for (int q = 0; q < kStageLoads; ++q) {
        const int idx = threadIdx.x + q * kPassBlock;
        const int i = idx >> 5, j = (idx >> 3) & 3, c4 = idx & 7;
        const int64_t e = (int64_t)ci * kChunk + c4 * 4;
        const bool ok = e < d;
        const float4 v = *reinterpret_cast<const float4*>(W + i * D + j * d + (ok ? e : 0));
        w[q] = ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// Splits (bf16) or copies (fp32) the fetched weights into LDS stage buffer `dst`
// (one buffer: kBf16Stage uint4 or kF32Stage floats).
template <bool kBf16>
__device__ __forceinline__ void commit_weights(void* dst, const float4 (&w)[kStageLoads]) {
#pragma unroll
    for (int q = 0; q < kStageLoads; ++q) {
        const int idx = threadIdx.x + q * kPassBlock;
        const int i = idx >> 5, j = (idx >> 3) & 3, c4 = idx & 7;
        if constexpr (kBf16) {
            const float wv[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
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
            // B operand of tile nt = i/16: lane (k-group = c4/2)*16 + column i%16,
            // 8 bf16 per lane of which this float4 fills half c4%2
            const int nt = i >> 4, col = i & 15;
            const int lane = (c4 >> 1) * 16 + col;
            const int half = c4 & 1;
            uint2* base = reinterpret_cast<uint2*>(dst);
            base[b_slot(0, nt, j, lane) * 2 + half] = make_uint2(hi[0], hi[1]);
            base[b_slot(1, nt, j, lane) * 2 + half] = make_uint2(mid[0], mid[1]);
            base[b_slot(2, nt, j, lane) * 2 + half] = make_uint2(lo[0], lo[1]);
        } else {
            // layout [32 rows][4 streams][32 channels], row stride kF32Row floats
            *reinterpret_cast<float4*>(static_cast<float*>(dst) + i * kF32Row + j * kChunk + c4 * 4) = w[q];
        }
    }
}

// Raw 8-element stream data of one lane for one step (registers only).
template <bool kBf16>
struct Raw8;
template <>
struct Raw8<true> {
    uint4 w;
    __device__ __forceinline__ void load(const void* base, int64_t idx) {
        w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    }
    __device__ __forceinline__ void zero() { w = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ void to(Vec8<true>& v) const {
        v.raw = w;
        v.unpack();
    }
};
template <>
struct Raw8<false> {
    float4 a, b;
    __device__ __forceinline__ void load(const void* base, int64_t idx) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
        a = p[0];
        b = p[1];
    }
    __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void to(Vec8<false>& v) const {
        v.v[0] = a.x; v.v[1] = a.y; v.v[2] = a.z; v.v[3] = a.w;
        v.v[4] = b.x; v.v[5] = b.y; v.v[6] = b.z; v.v[7] = b.w;
    }
};

template <bool kBf16, bool kPost>
struct StepData {
    Raw8<kBf16> x[kHC];
    Raw8<kBf16> f;  // used when kPost
};

// Loads one step's stream values of a lane. Out-of-range lanes (token >= n or
// channel >= d) load from token 0 / channel 0, which always exists, and get
// zeros, so the loads are unconditional.
template <bool kBf16, bool kPost>
__device__ __forceinline__ void load_step(StepData<kBf16, kPost>& s, const PassArgs& a, int64_t t, bool live,
                                          int64_t e) {
    const int64_t tt = live ? t : 0, ee = live ? e : 0;
#pragma unroll
    for (int j = 0; j < kHC; ++j) s.x[j].load(a.res, (tt * kHC + j) * a.d + ee);
    if constexpr (kPost) s.f.load(a.f, tt * a.d + ee);
    if (!live) {
#pragma unroll
        for (int j = 0; j < kHC; ++j) s.x[j].zero();
        if constexpr (kPost) s.f.zero();
    }
}

// Per-lane constant state of one sweep (one 16-token tile).
struct LaneCoef {
    float pk[kHC];        // previous sublayer's post (expand)
    float cm[kHC * kHC];  // previous sublayer's comb (expand)
    float pim[kHC];       // collapse weights
};

template <bool kPost, bool kPre>
__device__ __forceinline__ void load_coef(LaneCoef& co, const PassArgs& a, int64_t t, bool tok_ok) {
#pragma unroll
    for (int j = 0; j < kHC; ++j) co.pk[j] = co.pim[j] = 0.f;
#pragma unroll
    for (int i = 0; i < kHC * kHC; ++i) co.cm[i] = 0.f;
    if (!tok_ok) return;
    if constexpr (kPost) {
        const float4 pv = reinterpret_cast<const float4*>(a.post_prev)[t];
        co.pk[0] = pv.x; co.pk[1] = pv.y; co.pk[2] = pv.z; co.pk[3] = pv.w;
#pragma unroll
        for (int j = 0; j < kHC; ++j) {
            const float4 c = reinterpret_cast<const float4*>(a.comb_prev)[t * 4 + j];
            co.cm[4 * j] = c.x; co.cm[4 * j + 1] = c.y; co.cm[4 * j + 2] = c.z; co.cm[4 * j + 3] = c.w;
        }
    }
    if constexpr (kPre) {
        const float4 pv = reinterpret_cast<const float4*>(a.pre_mix)[t];
        co.pim[0] = pv.x; co.pim[1] = pv.y; co.pim[2] = pv.z; co.pim[3] = pv.w;
    }
}

// Elementwise part of one step for one tile: expand (optional), collapse
// (optional), sum of squares. Leaves the (rounded) stream values in xs.
template <bool kBf16, bool kPost, bool kPre>
__device__ __forceinline__ void step_elementwise(const PassArgs& a, const StepData<kBf16, kPost>& in,
                                                 const LaneCoef& co, int64_t t, bool live, int64_t e,
                                                 Vec8<kBf16> (&xs)[kHC], float& sumsq) {
    const int64_t d = a.d;
#pragma unroll
    for (int j = 0; j < kHC; ++j) in.x[j].to(xs[j]);
    if constexpr (kPost) {
        Vec8<kBf16> fv, x1[kHC];
        in.f.to(fv);
        expand8<kBf16>(fv, xs, co.pk, co.cm, x1);
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
            for (int j = 0; j < kHC; ++j) s = fmaf(co.pim[j], xs[j].v[c], s);
            yv.v[c] = s;
        }
        yv.round();
        if (live) yv.store(a.y, t * d + e);
    }
#pragma unroll
    for (int j = 0; j < kHC; ++j)
#pragma unroll
        for (int c = 0; c < 8; ++c) sumsq = fmaf(xs[j].v[c], xs[j].v[c], sumsq);
}

// The sweep: workgroup = 4 waves x kTiles tiles of 16 tokens. Per 32-channel step,
// each lane loads its tiles' stream values, fetches the next step's weights (L2)
// before doing the step's work, and after the step's MFMAs splits those weights
// into the other LDS buffer; one barrier per step. Every B fragment read from LDS
// feeds all kTiles tiles of the wave.
template <bool kBf16, bool kPost, bool kPre>
__global__ __launch_bounds__(kPassBlock) void pass_kernel(PassArgs a) {
    __shared__ PassLds<kBf16> lds;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int64_t n = a.n, d = a.d;
    const int split = (int)(blockIdx.x % (unsigned)a.nsplit);
    const int64_t group = blockIdx.x / (unsigned)a.nsplit;
    const int64_t tbase = group * kTokWG + wave * kTokWave;   // first token of the wave
    const int c_begin = split * a.chunks_per_split;
    const int c_end = min(a.nchunks, c_begin + a.chunks_per_split);

    // the B columns 24..31 (tile 1, columns 8..15) stay zero for the whole sweep
    if constexpr (kBf16) {
        for (int z = threadIdx.x; z < 2 * 3 * kHC * 4 * 8; z += kPassBlock) {
            const int col = 8 + (z & 7), gg = (z >> 3) & 3, j = (z >> 5) & 3, term = (z >> 7) % 3,
                      buf = z / (3 * kHC * 4 * 8);
            lds.b[buf][b_slot(term, 1, j, gg * 16 + col)] = make_uint4(0, 0, 0, 0);
        }
    } else {
        for (int z = threadIdx.x; z < 2 * 8 * kF32Row; z += kPassBlock) {
            const int buf = z / (8 * kF32Row), o = z - buf * 8 * kF32Row;
            lds.w[buf][kMix * kF32Row + o] = 0.f;
        }
    }

    int64_t t[kTiles];
    bool tok_ok[kTiles];
    LaneCoef co[kTiles];
    floatx4_t acc[kTiles][2];
    float sumsq[kTiles];
#pragma unroll
    for (int q = 0; q < kTiles; ++q) {
        t[q] = tbase + q * 16 + r;
        tok_ok[q] = t[q] < n;
        load_coef<kPost, kPre>(co[q], a, t[q], tok_ok[q]);
        acc[q][0] = acc[q][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        sumsq[q] = 0.f;
    }

    if (c_begin < c_end) {
        float4 w0[kStageLoads];
        fetch_weights(w0, a.hc_fn, d, c_begin);
        commit_weights<kBf16>(kBf16 ? (void*)lds_b(lds, 0) : (void*)lds_w(lds, 0), w0);
    }
    __syncthreads();

    for (int ci = c_begin; ci < c_end; ++ci) {
        const int buf = (ci - c_begin) & 1;
        const bool more = ci + 1 < c_end;
        float4 wnext[kStageLoads];
        if (more) fetch_weights(wnext, a.hc_fn, d, ci + 1);   // L2, committed after the MFMAs
        const int64_t e = (int64_t)ci * kChunk + g * 8;
        StepData<kBf16, kPost> in[kTiles];
#pragma unroll
        for (int q = 0; q < kTiles; ++q) load_step<kBf16, kPost>(in[q], a, t[q], tok_ok[q] && e < d, e);

        Vec8<kBf16> xs[kTiles][kHC];
#pragma unroll
        for (int q = 0; q < kTiles; ++q)
            step_elementwise<kBf16, kPost, kPre>(a, in[q], co[q], t[q], tok_ok[q] && e < d, e, xs[q], sumsq[q]);

        if constexpr (kBf16) {
            const uint4* B = lds.b[buf];
#pragma unroll
            for (int j = 0; j < kHC; ++j)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                    for (int term = 0; term < 3; ++term) {
                        const bf16x8_t Bv = __builtin_bit_cast(bf16x8_t, B[b_slot(term, nt, j, lane)]);
#pragma unroll
                        for (int q = 0; q < kTiles; ++q)
                            acc[q][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, xs[q][j].raw), Bv, acc[q][nt], 0, 0, 0);
                    }
        } else {
            // lane (r, g): A = token r, channel g*8 + c; B = mix nt*16 + r, same channel
            const float* W = lds.w[buf];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int j = 0; j < kHC; ++j) {
                    const float* wr = W + (nt * 16 + r) * kF32Row + j * kChunk + g * 8;
                    const float4 b0 = *reinterpret_cast<const float4*>(wr);
                    const float4 b1 = *reinterpret_cast<const float4*>(wr + 4);
                    const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                    for (int c = 0; c < 8; ++c)
#pragma unroll
                        for (int q = 0; q < kTiles; ++q)
                            acc[q][nt] =
                                __builtin_amdgcn_mfma_f32_16x16x4f32(xs[q][j].v[c], bv[c], acc[q][nt], 0, 0, 0);
                }
        }
        // the other buffer was last read before the previous barrier
        if (more) commit_weights<kBf16>(kBf16 ? (void*)lds_b(lds, buf ^ 1) : (void*)lds_w(lds, buf ^ 1), wnext);
        __syncthreads();
    }

    // partial results of this (token group, channel slice)
    float* part = a.part + (int64_t)split * n * kPart;
#pragma unroll
    for (int q = 0; q < kTiles; ++q) {
        float s = sumsq[q];
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        if (g == 0 && tok_ok[q]) part[t[q] * kPart + kMix] = s;
        // accumulator layout: lane holds rows 4*g .. 4*g+3 (tokens), column r (mix)
        const int64_t t0 = tbase + q * 16 + 4 * g;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int mix = nt * 16 + r;
            if (mix < kMix) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    if (t0 + ii < n) part[(t0 + ii) * kPart + mix] = acc[q][nt][ii];
            }
        }
    }
}

// ------------------------------------------------------------------ finalize
// 16 lanes per token (a 64-lane wave holds 4 tokens). Lane e owns partial
// entries e and 16 + e (dots 0..23, sum of squares at 24) and, in the split,
// comb entry C[e/4][e%4]; lanes 0..3 also own pre[e], lanes 4..7 post[e-4]. Row
// sums combine lanes of a quad, column sums lanes 4 apart (DPP, no LDS).

// DPP lane exchanges inside a row of 16 lanes:
// quad_perm [1,0,3,2] / [2,3,0,1] swap neighbours / pairs, row_ror:n rotates by n.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}
constexpr int kQuadSwap1 = 0xb1, kQuadSwap2 = 0x4e, kRowRor4 = 0x124, kRowRor8 = 0x128;

__device__ __forceinline__ float row_sum16(float v) {   // lanes 4r..4r+3
    v += dpp<kQuadSwap1>(v);
    return v + dpp<kQuadSwap2>(v);
}
__device__ __forceinline__ float col_sum16(float v) {   // lanes k, k+4, k+8, k+12
    v += dpp<kRowRor8>(v);
    return v + dpp<kRowRor4>(v);
}

struct FinalizeArgs {
    const float* part;     // [nsplit][n][kPart]
    int nsplit;
    int64_t n;
    int64_t D;             // hc * d
    float norm_eps;
    const float* scale;    // split only
    const float* base;
    int iters;
    float eps;
    bool split;
    float* mixes;          // nullable
    float* pre;
    float* post;
    float* comb;
};

// Token t (shared by the 16-lane group; t >= n: computes on token 0, stores
// nothing), lane e of the group. Every lane of the wave must call it.
__device__ __forceinline__ void finalize16(const FinalizeArgs& f, int64_t t, int e) {
    const bool ok = t < f.n;
    const int64_t tt = ok ? t : 0;
    // fixed-order reduction over the channel slices
    float a0 = 0.f, a1 = 0.f;
    for (int s = 0; s < f.nsplit; ++s) {
        const float* p = f.part + ((int64_t)s * f.n + tt) * kPart;
        a0 += p[e];
        a1 += p[16 + e];                   // entries 16..31; 25..31 are never used below
    }
    const int lane16 = (threadIdx.x & 63) & ~15;
    const float sumsq = __shfl(a1, lane16 + (kMix - 16));
    const float rstd = 1.0f / sqrtf(sumsq / (float)f.D + f.norm_eps);
    const float m0 = a0 * rstd;            // mixes[e]
    const float m1 = a1 * rstd;            // mixes[16 + e] (valid for e < 8)
    if (f.mixes && ok) {
        f.mixes[t * kMix + e] = m0;
        if (e < kMix - 16) f.mixes[t * kMix + 16 + e] = m1;
    }
    if (!f.split) return;                  // uniform
    // comb logit of entry e is mixes[8 + e]: lane 8+e's m0 for e < 8, lane e-8's m1 otherwise
    const float lo = __shfl(m0, lane16 + ((8 + e) & 15));
    const float hi = __shfl(m1, lane16 + ((e + 8) & 15));
    const float m = e < 8 ? lo : hi;
    float c = m * f.scale[2] + f.base[8 + e];
    // row softmax (max subtracted), + eps
    float mx = fmaxf(c, dpp<kQuadSwap1>(c));
    mx = fmaxf(mx, dpp<kQuadSwap2>(mx));
    c = __expf(c - mx);
    c = c * __builtin_amdgcn_rcpf(row_sum16(c)) + f.eps;
    c *= __builtin_amdgcn_rcpf(col_sum16(c) + f.eps);
    for (int it = 1; it < f.iters; ++it) {
        c *= __builtin_amdgcn_rcpf(row_sum16(c) + f.eps);
        c *= __builtin_amdgcn_rcpf(col_sum16(c) + f.eps);
    }
    if (ok) {
        f.comb[t * 16 + e] = c;
        if (e < kHC) f.pre[t * kHC + e] = sigmoid(m0 * f.scale[0] + f.base[e]) + f.eps;
        else if (e < 2 * kHC) f.post[t * kHC + e - kHC] = 2.0f * sigmoid(m0 * f.scale[1] + f.base[e]);
    }
}

constexpr int kFinBlock = 256;

__global__ __launch_bounds__(kFinBlock) void finalize_kernel(FinalizeArgs f) {
    finalize16(f, ((int64_t)blockIdx.x * kFinBlock + threadIdx.x) >> 4, threadIdx.x & 15);
}

// ------------------------------------------------- bf16 sweep (stream-stationary)
// Loading in the MFMA operand layout (16 token rows x 64 B per instruction) caps
// reads at ~3.9 TB/s on MI355X, while 256-byte row runs reach ~5.8 TB/s, so
// streams are loaded rowwise and transposed through LDS:
//   - workgroup = 4 waves x 16 tokens; super-step = 128 channels. Lane
//     (sub = lane/16, ch = lane%16) of wave w loads, for token group G (4 per
//     wave) and stream j, 16 B at token 16w + 4G + sub, channels cs + 8ch: one
//     instruction = 4 tokens x 256 B. Expand / collapse / sum of squares run in
//     that layout (stores are 256 B runs too).
//   - every wave writes its rounded values, all 4 streams, into the shared LDS
//     A region in MFMA A layout (row = token, k-group = 8 channels),
//     XOR-swizzled so that writes and reads are free of bank conflicts.
//   - in the MFMA phase wave w owns stream j = w for all 64 tokens (4 row tiles).
//     Its B operands come from L2, one 16-byte load per lane each, from weights
//     split once per call (pack_weights_kernel) into three bf16 terms (hi + mid
//     + lo, ~24 significant bits). The 24 mix columns take 5 MFMAs per tile and
//     k-block (no zero padding): column tile 0 = mixes 0..15 (hi, mid, lo into
//     one accumulator); column tile 1 = [hi | mid] of mixes 16..23, then [lo | 0]
//     of mixes 16..23 into the same accumulator, whose two 8-column halves are
//     added once at the end. A sixth MFMA multiplies the A tile by itself: since
//     the A and B lane layouts coincide, mfma(A, A) accumulates the tile's Gram
//     matrix, whose diagonal is each token's sum of squares. The 4 waves'
//     partial results (one stream each) are summed through LDS.
//   - two barriers per super-step; the next super-step's stream loads are issued
//     before the MFMA phase, so they overlap it.
constexpr int kSuper = 128;              // channels per super-step
constexpr int kKbPerSuper = kSuper / kChunk;
constexpr int kCoefF4 = 6;               // float4 per token: post_prev, comb_prev x4, pre_mix
constexpr int kFragsPerKb = 5;           // B operands per (stream, k-block): hi0 mid0 lo0 [hi1|mid1] [lo1|0]

struct Sweep2Lds {
    uint4 a[kHC * kKbPerSuper * 4 * 64];   // [stream][k-block][row tile][lane], 64 KB
    float4 coef[kTokWG][kCoefF4];         // 6 KB
};

// Swizzled A slot: slot = ((j*4 + kb)*4 + tile)*64 + g*16 + r. The low 3 bits are
// XORed with (g + 4*(kb & 1)): a transposing write (lanes with the same token
// group and stream spread over 2 k-blocks x 4 k-groups) and a lane-ordered read
// both touch 8 distinct bank groups per 8 lanes.
__device__ __forceinline__ int a2_slot(int j, int kb, int tile, int lane) {
    const int slot = ((j * kKbPerSuper + kb) * 4 + tile) * 64 + lane;
    return slot ^ (((lane >> 4) + 4 * (kb & 1)) & 7);
}

// Splits 8 fp32 weights into three bf16 terms (w ~ hi + mid + lo).
__device__ __forceinline__ void split3(const float4& a, const float4& b, uint4& hi, uint4& mid, uint4& lo) {
    const float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[4], m[4], l[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float x0 = w[2 * q], x1 = w[2 * q + 1];
        h[q] = pack_bf16x2(x0, x1);
        const float r0 = x0 - bf16_lo(h[q]), r1 = x1 - bf16_hi(h[q]);
        m[q] = pack_bf16x2(r0, r1);
        l[q] = pack_bf16x2(r0 - bf16_lo(m[q]), r1 - bf16_hi(m[q]));
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    mid = make_uint4(m[0], m[1], m[2], m[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// Packed weights: for stream j and 32-channel k-block kbg, 5 B operands of 64
// lanes x 16 B in v_mfma_f32_16x16x32_bf16 layout (lane: k-group g = lane/16,
// column col = lane%16, channels kbg*32 + 8g .. +8 of stream j):
//   0, 1, 2: hi, mid, lo of row col (mixes 0..15)
//   3: hi of row 16 + col (col < 8), mid of row 16 + col - 8 (col >= 8)
//   4: lo of row 16 + col (col < 8), zero (col >= 8)
// Channels >= d are zero. One thread per (j, kbg, lane).
__global__ __launch_bounds__(256) void pack_weights_kernel(const float* __restrict__ W, int64_t d, int nkb,
                                                           uint4* __restrict__ packed) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (int64_t)kHC * nkb * 64) return;
    const int lane = (int)(gid & 63);
    const int64_t jk = gid >> 6;                                    // j * nkb + kbg
    const int j = (int)(jk / nkb), kbg = (int)(jk - (int64_t)j * nkb);
    const int g = lane >> 4, col = lane & 15;
    const int64_t e0 = (int64_t)kbg * kChunk + g * 8;
    float4 w0a = make_float4(0.f, 0.f, 0.f, 0.f), w0b = w0a, w1a = w0a, w1b = w0a;
    if (e0 < d) {                                                   // d % 8 == 0: whole groups
        const float4* r0 = reinterpret_cast<const float4*>(W + (int64_t)col * kHC * d + (int64_t)j * d + e0);
        const float4* r1 =
            reinterpret_cast<const float4*>(W + (int64_t)(16 + (col & 7)) * kHC * d + (int64_t)j * d + e0);
        w0a = r0[0];
        w0b = r0[1];
        w1a = r1[0];
        w1b = r1[1];
    }
    uint4 h0, m0, l0, h1, m1, l1;
    split3(w0a, w0b, h0, m0, l0);
    split3(w1a, w1b, h1, m1, l1);
    uint4* dst = packed + jk * kFragsPerKb * 64 + lane;
    dst[0 * 64] = h0;
    dst[1 * 64] = m0;
    dst[2 * 64] = l0;
    const bool lo_half = col < 8;
    dst[3 * 64] = make_uint4(lo_half ? h1.x : m1.x, lo_half ? h1.y : m1.y, lo_half ? h1.z : m1.z,
                             lo_half ? h1.w : m1.w);
    dst[4 * 64] = make_uint4(lo_half ? l1.x : 0u, lo_half ? l1.y : 0u, lo_half ? l1.z : 0u, lo_half ? l1.w : 0u);
}

template <bool kPost, bool kPre>
__global__ __launch_bounds__(kPassBlock, 2) void sweep2_kernel(PassArgs a, const uint4* __restrict__ packed) {
    static_assert(kTokWave == 16 && kWaves == kHC, "one 16-token tile and one stream per wave");
    __shared__ Sweep2Lds lds;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane >> 4, ch = lane & 15;   // rowwise role
    const int64_t n = a.n, d = a.d;
    const int nkb = a.nchunks;
    const int split = (int)(blockIdx.x % (unsigned)a.nsplit);
    const int64_t group = blockIdx.x / (unsigned)a.nsplit;
    const int64_t tbase = group * kTokWG + wave * kTokWave;   // this wave's rowwise tokens
    const int kb_begin = split * a.chunks_per_split;
    const int kb_end = min(nkb, kb_begin + a.chunks_per_split);

    for (int z = threadIdx.x; z < kTokWG * kCoefF4; z += kPassBlock) {
        const int tl = z / kCoefF4, q = z - tl * kCoefF4;
        const int64_t tt = group * kTokWG + tl;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tt < n) {
            if (kPost && q == 0) v = reinterpret_cast<const float4*>(a.post_prev)[tt];
            if (kPost && q >= 1 && q <= 4) v = reinterpret_cast<const float4*>(a.comb_prev)[tt * 4 + q - 1];
            if (kPre && q == 5) v = reinterpret_cast<const float4*>(a.pre_mix)[tt];
        }
        lds.coef[tl][q] = v;
    }

    // buffer resources based at the wave's first token; ranges end at token n
    const int64_t row_x = kHC * d * 2, row_f = d * 2;   // bytes per token
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const char*>(a.res) + tbase * row_x, (n - tbase) * row_x);
    const __amdgpu_buffer_rsrc_t rf = make_rsrc(kPost ? static_cast<const char*>(a.f) + tbase * row_f : nullptr,
                                                kPost ? (n - tbase) * row_f : 0);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(kPost ? static_cast<char*>(a.streams_out) + tbase * row_x : nullptr,
                                                kPost ? (n - tbase) * row_x : 0);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(kPre ? static_cast<char*>(a.y) + tbase * row_f : nullptr,
                                                kPre ? (n - tbase) * row_f : 0);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(packed, (int64_t)kHC * nkb * kFragsPerKb * 64 * 16);
    const uint32_t lane_x = (uint32_t)(sub * row_x + ch * 16);
    const uint32_t lane_f = (uint32_t)(sub * row_f + ch * 16);
    const uint32_t lane_p = (uint32_t)(lane * 16);
    const int g = lane >> 4, col = lane & 15;   // MFMA role: k-group, column

    floatx4_t acc[4][2], gram[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q][0] = acc[q][1] = gram[q] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    Raw8<true> X[4][kHC], F[4];
    auto load_x = [&](int kb0) {
        const int64_t cs = (int64_t)kb0 * kChunk, c = cs + ch * 8;
        const bool c_ok = c < d && c < (int64_t)kb_end * kChunk;
#pragma unroll
        for (int G = 0; G < 4; ++G) {
            const bool live = c_ok && tbase + 4 * G + sub < n;   // masked lanes read zeros
            const uint32_t vx = live ? lane_x : kOffMasked, vf = live ? lane_f : kOffMasked;
#pragma unroll
            for (int j = 0; j < kHC; ++j)
                X[G][j].w = buf_load16(rx, vx, (uint32_t)((4 * G * kHC + j) * row_f + cs * 2));
            if constexpr (kPost) F[G].w = buf_load16(rf, vf, (uint32_t)(4 * G * row_f + cs * 2));
        }
    };
    // B operands of the next k-block to multiply (one k-block ahead, carried
    // across super-steps so the elementwise phase hides their latency)
    uint4 Bf[kFragsPerKb];
    auto load_b = [&](int kbg) {
        if (kbg < kb_end) {
#pragma unroll
            for (int q = 0; q < kFragsPerKb; ++q)
                Bf[q] = buf_load16(rp, lane_p, (uint32_t)((((int64_t)wave * nkb + kbg) * kFragsPerKb + q) * 64 * 16));
        }
    };
    if (kb_begin < kb_end) load_x(kb_begin);
    load_b(kb_begin);
    __syncthreads();   // coefficients

    for (int kb0 = kb_begin; kb0 < kb_end; kb0 += kKbPerSuper) {
        const int64_t cs = (int64_t)kb0 * kChunk, c = cs + ch * 8;
        const bool c_ok = c < d && c < (int64_t)kb_end * kChunk;
        // expand / collapse / sum of squares, rowwise, two channels (one packed
        // word per stream) at a time; results into the A region
#pragma unroll
        for (int G = 0; G < 4; ++G) {
            const bool live = c_ok && tbase + 4 * G + sub < n;
            const uint32_t vx = live ? lane_x : kOffMasked, vf = live ? lane_f : kOffMasked;
            const float4* cf = lds.coef[wave * kTokWave + 4 * G + sub];
            float pk[kHC], cm[kHC * kHC], pim[kHC];
            if constexpr (kPost) {
                const float4 pv = cf[0];
                pk[0] = pv.x; pk[1] = pv.y; pk[2] = pv.z; pk[3] = pv.w;
#pragma unroll
                for (int j = 0; j < kHC; ++j) {
                    const float4 cv = cf[1 + j];
                    cm[4 * j] = cv.x; cm[4 * j + 1] = cv.y; cm[4 * j + 2] = cv.z; cm[4 * j + 3] = cv.w;
                }
            }
            if constexpr (kPre) {
                const float4 pv = cf[5];
                pim[0] = pv.x; pim[1] = pv.y; pim[2] = pv.z; pim[3] = pv.w;
            }
            uint32_t yw[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t xw[kHC];
#pragma unroll
                for (int j = 0; j < kHC; ++j) xw[j] = (&X[G][j].w.x)[w];
                if constexpr (kPost) {
                    const uint32_t fw = (&F[G].w.x)[w];
                    const float f0 = bf16_lo(fw), f1 = bf16_hi(fw);
                    uint32_t ow[kHC];
#pragma unroll
                    for (int k = 0; k < kHC; ++k) {
                        float o0 = pk[k] * f0, o1 = pk[k] * f1;
#pragma unroll
                        for (int j = 0; j < kHC; ++j) {
                            o0 = fmaf(cm[4 * j + k], bf16_lo(xw[j]), o0);
                            o1 = fmaf(cm[4 * j + k], bf16_hi(xw[j]), o1);
                        }
                        ow[k] = pack_bf16x2(o0, o1);
                    }
#pragma unroll
                    for (int k = 0; k < kHC; ++k) xw[k] = (&X[G][k].w.x)[w] = ow[k];
                }
                if constexpr (kPre) {
                    float y0 = 0.f, y1 = 0.f;
#pragma unroll
                    for (int j = 0; j < kHC; ++j) {
                        y0 = fmaf(pim[j], bf16_lo(xw[j]), y0);
                        y1 = fmaf(pim[j], bf16_hi(xw[j]), y1);
                    }
                    yw[w] = pack_bf16x2(y0, y1);
                }
            }
            if constexpr (kPost) {
#pragma unroll
                for (int k = 0; k < kHC; ++k)
                    buf_store16(X[G][k].w, ro, vx, (uint32_t)((4 * G * kHC + k) * row_f + cs * 2));
            }
            if constexpr (kPre)
                buf_store16(make_uint4(yw[0], yw[1], yw[2], yw[3]), ry, vf, (uint32_t)(4 * G * row_f + cs * 2));
            // A layout: tile = wave, row = 4G + sub, k-block = ch / 4, k-group = ch % 4
#pragma unroll
            for (int j = 0; j < kHC; ++j)
                lds.a[a2_slot(j, ch >> 2, wave, (ch & 3) * 16 + 4 * G + sub)] = X[G][j].w;
            __builtin_amdgcn_sched_barrier(0);
        }
        // next super-step's streams: in flight during the MFMA phase
        if (kb0 + kKbPerSuper < kb_end) load_x(kb0 + kKbPerSuper);
        __syncthreads();   // A region complete

        // MFMA phase: stream j = wave, 4 row tiles, the super-step's k-blocks; once a
        // k-block's MFMAs are issued its B registers take the next k-block
#pragma unroll 1
        for (int k = 0; k < kKbPerSuper; ++k) {
            const int kbg = kb0 + k;
            if (kbg >= kb_end) break;   // uniform
#pragma unroll
            for (int tile = 0; tile < 4; ++tile) {
                const bf16x8_t A = __builtin_bit_cast(bf16x8_t, lds.a[a2_slot(wave, k, tile, lane)]);
#pragma unroll
                for (int q = 0; q < kFragsPerKb; ++q)
                    acc[tile][q < 3 ? 0 : 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        A, __builtin_bit_cast(bf16x8_t, Bf[q]), acc[tile][q < 3 ? 0 : 1], 0, 0, 0);
                gram[tile] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, A, gram[tile], 0, 0, 0);
            }
            load_b(kbg + 1);
        }
        __syncthreads();   // A region consumed
    }

    float* part = a.part + (int64_t)split * n * kPart;
    // column tile 1: mixes 16 + c = columns c ([hi | lo] part) + c + 8 ([mid] part)
#pragma unroll
    for (int tile = 0; tile < 4; ++tile)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) acc[tile][1][ii] += dpp<kRowRor8>(acc[tile][1][ii]);
    // partial projections and sums of squares (Gram diagonal: row 4g + ii sits in
    // column 4g + ii) of the 4 streams: sum over waves through LDS
    float* red = reinterpret_cast<float*>(lds.a);   // [wave][tile][nt][ii][lane], 32 KB
    float* red_ss = red + kWaves * 2048;            // [wave][tile][row], 1 KB
#pragma unroll
    for (int tile = 0; tile < 4; ++tile)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) red[(((wave * 4 + tile) * 2 + nt) * 4 + ii) * 64 + lane] = acc[tile][nt][ii];
#pragma unroll
    for (int tile = 0; tile < 4; ++tile)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            if (col == 4 * g + ii) red_ss[(wave * 4 + tile) * 16 + col] = gram[tile][ii];
    __syncthreads();
    for (int e = threadIdx.x; e < 4 * 2 * 4 * 64; e += kPassBlock) {
        const int l = e & 63, ii = (e >> 6) & 3, nt = (e >> 8) & 1, tile = e >> 9;
        const int mix = nt * 16 + (l & 15);
        const int64_t t = group * kTokWG + tile * 16 + 4 * (l >> 4) + ii;
        if (mix < kMix && t < n) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) s += red[w * 2048 + e];
            part[t * kPart + mix] = s;
        }
    }
    if (threadIdx.x < kTokWG) {   // token tile*16 + row of the group
        const int tile = threadIdx.x >> 4, row = threadIdx.x & 15;
        const int64_t t = group * kTokWG + threadIdx.x;
        if (t < n) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) s += red_ss[(w * 4 + tile) * 16 + row];
            part[t * kPart + kMix] = s;
        }
    }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// ------------------------------------------------------------------- launchers
PassPlan plan_pass(int64_t n, int64_t d) {
    PassPlan p{};
    p.tiles = ceil_div(n, kTokWG);
    p.nchunks = (int)ceil_div(d, kChunk);
    // channel slices are whole 128-channel super-steps (the bf16 sweep's unit)
    const int nsuper = (int)ceil_div(d, kSuper);
    const int64_t target_groups = HC_TARGET_GROUPS;
    int64_t ns = ceil_div(target_groups, p.tiles > 0 ? p.tiles : 1);
    if (ns < 1) ns = 1;
    if (ns > nsuper) ns = nsuper;
    if (ns > 64) ns = 64;
    p.chunks_per_split = (int)ceil_div(nsuper, ns) * kKbPerSuper;
    p.nsplit = (int)ceil_div(p.nchunks, p.chunks_per_split);
    // [partial rows: nsplit x n x 32 floats][packed weights: 4 streams x nchunks x 5 x 1 KB]
    p.partial_bytes = (size_t)p.nsplit * (size_t)n * kPart * sizeof(float);
    p.packed_bytes = (size_t)kHC * (size_t)p.nchunks * kFragsPerKb * 64 * 16;
    p.workspace_bytes = p.partial_bytes + p.packed_bytes;
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
template <bool kPost, bool kPre>
void launch_sweep2_t(const PassArgs& a, const PassPlan& p, const uint4* packed, hipStream_t stream) {
    hipLaunchKernelGGL((sweep2_kernel<kPost, kPre>), dim3((unsigned)(p.tiles * p.nsplit)), dim3(kPassBlock), 0,
                       stream, a, packed);
}

template <bool kPost, bool kPre>
void launch_pass_t(const PassArgs& a, const PassPlan& p, hipStream_t stream) {
    hipLaunchKernelGGL((pass_kernel<false, kPost, kPre>), dim3((unsigned)(p.tiles * p.nsplit)), dim3(kPassBlock), 0,
                       stream, a);
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
    a.nsplit = p.nsplit;
    FinalizeArgs f{};
    f.part = a.part;
    f.nsplit = p.nsplit;
    f.n = r.n;
    f.D = r.d * kHC;
    f.norm_eps = r.norm_eps;
    f.scale = r.scale;
    f.base = r.base;
    f.iters = r.iters;
    f.eps = r.eps;
    f.split = r.split;
    f.mixes = r.mixes;
    f.pre = r.pre;
    f.post = r.post;
    f.comb = r.comb;
    const bool post = r.f_prev != nullptr, pre = r.y != nullptr;
    if (r.bf16) {
        // weights split into bf16 terms in MFMA B layout, once per call
        uint4* packed = reinterpret_cast<uint4*>(static_cast<char*>(r.workspace) + p.partial_bytes);
        hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)ceil_div((int64_t)kHC * p.nchunks * 64, 256)),
                           dim3(256), 0, stream, r.hc_fn, r.d, p.nchunks, packed);
        if (post && pre) launch_sweep2_t<true, true>(a, p, packed, stream);
        else if (post) launch_sweep2_t<true, false>(a, p, packed, stream);
        else if (pre) launch_sweep2_t<false, true>(a, p, packed, stream);
        else launch_sweep2_t<false, false>(a, p, packed, stream);
    } else {
        if (post && pre) launch_pass_t<true, true>(a, p, stream);
        else if (post) launch_pass_t<true, false>(a, p, stream);
        else if (pre) launch_pass_t<false, true>(a, p, stream);
        else launch_pass_t<false, false>(a, p, stream);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)ceil_div(r.n * 16, kFinBlock)), dim3(kFinBlock), 0, stream, f);
    return hipGetLastError();
}

}  // namespace hc
