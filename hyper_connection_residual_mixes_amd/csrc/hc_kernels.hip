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
//   bf16_sweep_kernel   one pass over 64 tokens x a channel slice of bf16 streams
//                       (bf16_sweep2_kernel: 128 tokens, for large n):
//                       optional expand (previous sublayer's post/comb), optional
//                       collapse, and the partial 24-wide projection (MFMA) and
//                       sum of squares of the (rounded) streams, to a workspace.
//   pass_kernel         the same pass for fp32 streams (fp32 MFMA).
//   finalize_kernel     16 lanes per token: reduce the slice partials in a fixed
//                       order, scale by the RMS statistic, and (optionally) split.
//   finalize_wave_kernel the same with a wave per token, for many slices.
//   rmsnorm_mxfp8_kernel the sublayer RMSNorm (learned gain) of the collapsed
//                       input and its MXFP8 cast, a wave per token row.
//
// Stream counts other than four run the kernels of hc_generic.hip.
//
// All arithmetic is fp32 (MFMA products exact, fp32 accumulation). bf16 values
// are rounded to nearest-even (v_cvt_pk_bf16_f32).
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
constexpr int kWaves = 4;           // waves per fp32 pass workgroup
constexpr int kTiles = 1;           // 16-token MFMA row tiles per wave (fp32 pass)
constexpr int kPassTargetGroups = 512;
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
// The scalar offset must be wave-uniform; readfirstlane states that to the
// compiler, which otherwise may keep it in a vector register and wrap the access
// in a loop over its distinct values.
__device__ __forceinline__ int uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, uniform(soff), 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 buf_load16f(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, uniform(soff), 0);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
// A 16-byte store reads its data registers after issue. Nothing may overwrite
// them in the next two cycles; the compiler does not keep that distance here
// (a write to the first data register right after the store was seen to corrupt
// stored values), so every such store is followed by two wait states that no
// instruction is scheduled into.
__device__ __forceinline__ void buf_store16(uint4 v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, (int)voff, uniform(soff), 0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 1");
    __builtin_amdgcn_sched_barrier(0);
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
// (wave-uniform addresses: scalar loads). The Sinkhorn normalisations run in
// factored form: after the first round's row softmax + eps gives K, every later
// matrix is diag(r) K diag(c), and dividing row j by its sum + eps is the update
// r_j <- r_j / (r_j (K c)_j + eps) (columns likewise with K^T r). That is 56 VALU
// operations per round instead of 72 for rescaling all 16 entries; C = r_j K_jk c_k
// is formed once at the end. Each division multiplies by a reciprocal of
// (sum + eps) computed once per row or column.
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
    float K[kHC * kHC];
#pragma unroll
    for (int i = 0; i < kHC * kHC; ++i) K[i] = m[2 * kHC + i] * s2 + base[2 * kHC + i];
    // first round: row softmax (max subtracted), + eps
#pragma unroll
    for (int j = 0; j < kHC; ++j) {
        float mx = fmaxf(fmaxf(K[4 * j], K[4 * j + 1]), fmaxf(K[4 * j + 2], K[4 * j + 3]));
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            K[4 * j + k] = __expf(K[4 * j + k] - mx);
            s += K[4 * j + k];
        }
        const float inv = __builtin_amdgcn_rcpf(s);
#pragma unroll
        for (int k = 0; k < kHC; ++k) K[4 * j + k] = K[4 * j + k] * inv + eps;
    }
    float r[kHC], c[kHC];
#pragma unroll
    for (int j = 0; j < kHC; ++j) r[j] = c[j] = 1.0f;
    auto cols = [&]() {
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            float v = K[k] * r[0];
#pragma unroll
            for (int j = 1; j < kHC; ++j) v = fmaf(K[4 * j + k], r[j], v);
            c[k] *= __builtin_amdgcn_rcpf(fmaf(c[k], v, eps));
        }
    };
    auto rows = [&]() {
#pragma unroll
        for (int j = 0; j < kHC; ++j) {
            float u = K[4 * j] * c[0];
#pragma unroll
            for (int k = 1; k < kHC; ++k) u = fmaf(K[4 * j + k], c[k], u);
            r[j] *= __builtin_amdgcn_rcpf(fmaf(r[j], u, eps));
        }
    };
    cols();
    for (int it = 1; it < iters; ++it) {
        rows();
        cols();
    }
#pragma unroll
    for (int j = 0; j < kHC; ++j)
#pragma unroll
        for (int k = 0; k < kHC; ++k) C[4 * j + k] = r[j] * K[4 * j + k] * c[k];
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

// kStream: the outputs are written with non-temporal stores, which go to HBM
// without being kept in the caches. Chosen for outputs far larger than the
// caches, where keeping them would only defer their write-back into the next
// kernel's reads.
template <bool kBf16, bool kStream>
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
    for (int k = 0; k < kHC; ++k) {
        if constexpr (kStream && kBf16) {
            __builtin_nontemporal_store(u32x4_t{ov[k].raw.x, ov[k].raw.y, ov[k].raw.z, ov[k].raw.w},
                                        reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(out) + (t * kHC + k) * d + e));
        } else if constexpr (kStream) {
            u32x4_t* q = reinterpret_cast<u32x4_t*>(static_cast<float*>(out) + (t * kHC + k) * d + e);
            const float* v = ov[k].v;
            __builtin_nontemporal_store(u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                                __float_as_uint(v[3])}, q);
            __builtin_nontemporal_store(u32x4_t{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                                                __float_as_uint(v[7])}, q + 1);
        } else {
            ov[k].store(out, (t * kHC + k) * d + e);
        }
    }
}

// ------------------------------------------------------ fp32 stream pass
// Workgroup = 4 waves x 16 tokens. Lane (r = lane % 16, g = lane / 16) of wave w
// owns token tile*64 + w*16 + r and, at sweep step ci, channels ci*32 + g*8 ..+8
// of all 4 streams. The step's slice of hc_fn (24 rows x 4 streams x 32 channels)
// is staged in LDS once per workgroup and shared by its 4 waves.
//
// Projection: v_mfma_f32_16x16x4f32 (A = 16 tokens x 4 channels, B = 4 channels
// x 16 mixes, exact fp32 products, fp32 accumulators) with k running over the 4
// lane groups, one MFMA per (stream, channel, column tile); the 24 mixes use two
// 16-wide column tiles whose columns 24..31 are zero.
//
// Pipelining: while step ci is computed, the weights of step ci+1 are fetched
// from L2 and copied into the other LDS buffer after step ci's MFMAs, then one
// barrier per step.
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

// A kernel's arguments are read by scalar loads that the compiler issues at
// their first use, so a use behind another load's wait costs one more memory
// round trip. Naming every field in an empty asm at entry has all of them
// issued together, with one wait.
__device__ __forceinline__ void pin_args(const PassArgs& a) {
    asm volatile("" ::"s"(a.res), "s"(a.f), "s"(a.post_prev), "s"(a.comb_prev), "s"(a.pre_mix), "s"(a.hc_fn),
                 "s"(a.streams_out), "s"(a.y), "s"(a.part), "s"(a.n), "s"(a.d), "s"(a.nchunks),
                 "s"(a.chunks_per_split), "s"(a.nsplit));
}

constexpr int kPassBlock = kWaves * 64;
constexpr int kF32Row = kHC * kChunk + 4;      // floats per mix row of the fp32 stage (padded)
constexpr int kF32Stage = 32 * kF32Row;        // floats per LDS buffer: 32 mix rows (24..31 zero)
constexpr int kStageLoads = (kMix * kHC * kChunk / 4) / kPassBlock;  // float4 per thread per step

struct PassLds {
    float w[2][kF32Stage];
};

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

// Copies the fetched weights into LDS stage buffer `dst`, laid out as
// [32 rows][4 streams][32 channels] with row stride kF32Row floats.
__device__ __forceinline__ void commit_weights(float* dst, const float4 (&w)[kStageLoads]) {
#pragma unroll
    for (int q = 0; q < kStageLoads; ++q) {
        const int idx = threadIdx.x + q * kPassBlock;
        const int i = idx >> 5, j = (idx >> 3) & 3, c4 = idx & 7;
        *reinterpret_cast<float4*>(dst + i * kF32Row + j * kChunk + c4 * 4) = w[q];
    }
}

// Eight fp32 stream values of one lane for one step (registers only).
struct Raw8 {
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

template <bool kPost>
struct StepData {
    Raw8 x[kHC];
    Raw8 f;  // used when kPost
};

// Loads one step's stream values of a lane. Out-of-range lanes (token >= n or
// channel >= d) load from token 0 / channel 0, which always exists, and get
// zeros, so the loads are unconditional.
template <bool kPost>
__device__ __forceinline__ void load_step(StepData<kPost>& s, const PassArgs& a, int64_t t, bool live,
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
template <bool kPost, bool kPre>
__device__ __forceinline__ void step_elementwise(const PassArgs& a, const StepData<kPost>& in,
                                                 const LaneCoef& co, int64_t t, bool live, int64_t e,
                                                 Vec8<false> (&xs)[kHC], float& sumsq) {
    const int64_t d = a.d;
#pragma unroll
    for (int j = 0; j < kHC; ++j) in.x[j].to(xs[j]);
    if constexpr (kPost) {
        Vec8<false> fv, x1[kHC];
        in.f.to(fv);
        expand8<false>(fv, xs, co.pk, co.cm, x1);
#pragma unroll
        for (int k = 0; k < kHC; ++k) {
            if (live) x1[k].store(a.streams_out, (t * kHC + k) * d + e);
            xs[k] = x1[k];
        }
    }
    if constexpr (kPre) {
        Vec8<false> yv;
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
    float ss = 0.f;   // this step's 32 squares, added to the running sum once
#pragma unroll
    for (int j = 0; j < kHC; ++j)
#pragma unroll
        for (int c = 0; c < 8; ++c) ss = fmaf(xs[j].v[c], xs[j].v[c], ss);
    sumsq += ss;
}

// The sweep: workgroup = 4 waves x kTiles tiles of 16 tokens. Per 32-channel step,
// each lane loads its tiles' stream values, fetches the next step's weights (L2)
// before doing the step's work, and after the step's MFMAs copies those weights
// into the other LDS buffer; one barrier per step.
template <bool kPost, bool kPre>
__global__ __launch_bounds__(kPassBlock) void pass_kernel(PassArgs a) {
    __shared__ PassLds lds;

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
    for (int z = threadIdx.x; z < 2 * 8 * kF32Row; z += kPassBlock) {
        const int buf = z / (8 * kF32Row), o = z - buf * 8 * kF32Row;
        lds.w[buf][kMix * kF32Row + o] = 0.f;
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
        commit_weights(lds.w[0], w0);
    }
    __syncthreads();

    for (int ci = c_begin; ci < c_end; ++ci) {
        const int buf = (ci - c_begin) & 1;
        const bool more = ci + 1 < c_end;
        float4 wnext[kStageLoads];
        if (more) fetch_weights(wnext, a.hc_fn, d, ci + 1);   // L2, committed after the MFMAs
        const int64_t e = (int64_t)ci * kChunk + g * 8;
        StepData<kPost> in[kTiles];
#pragma unroll
        for (int q = 0; q < kTiles; ++q) load_step<kPost>(in[q], a, t[q], tok_ok[q] && e < d, e);

        Vec8<false> xs[kTiles][kHC];
#pragma unroll
        for (int q = 0; q < kTiles; ++q)
            step_elementwise<kPost, kPre>(a, in[q], co[q], t[q], tok_ok[q] && e < d, e, xs[q], sumsq[q]);

        {
            // lane (r, g): A = token r, channel g*8 + c; B = mix nt*16 + r, same channel.
            // The step's 128 products per dot go to a fresh accumulator that is added to
            // the running one once: accumulation chains stay one step long, so the
            // rounding error does not grow with the slice length.
            const float* W = lds.w[buf];
            floatx4_t sacc[kTiles][2];
#pragma unroll
            for (int q = 0; q < kTiles; ++q) sacc[q][0] = sacc[q][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
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
                            sacc[q][nt] =
                                __builtin_amdgcn_mfma_f32_16x16x4f32(xs[q][j].v[c], bv[c], sacc[q][nt], 0, 0, 0);
                }
#pragma unroll
            for (int q = 0; q < kTiles; ++q) {
                acc[q][0] += sacc[q][0];
                acc[q][1] += sacc[q][1];
            }
        }
        // the other buffer was last read before the previous barrier
        if (more) commit_weights(lds.w[buf ^ 1], wnext);
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

__device__ __forceinline__ void pin_args(const FinalizeArgs& f) {
    asm volatile("" ::"s"(f.part), "s"(f.nsplit), "s"(f.n), "s"(f.D), "s"(f.norm_eps), "s"(f.scale), "s"(f.base),
                 "s"(f.iters), "s"(f.eps), "s"((int)f.split), "s"(f.mixes), "s"(f.pre), "s"(f.post), "s"(f.comb));
}

// The split parameters lane e of a 16-lane group needs, fetched before the
// partial rows so that both are in flight together.
struct CoefParams {
    float s0, s1, s2, b_e, b_8e;   // hc_scale[0..2], hc_base[e], hc_base[8 + e]
};
// Raw buffer loads with empty ranges when there is no split (they return zeros):
// no branch, so they are issued with the partial rows' loads instead of after a
// wait for the parameter pointers.
__device__ __forceinline__ float buf_load4f(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0));
}
__device__ __forceinline__ CoefParams load_coef_params(const FinalizeArgs& f, int e) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(f.split ? f.scale : nullptr, f.split ? 3 * 4 : 0);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(f.split ? f.base : nullptr, f.split ? kMix * 4 : 0);
    CoefParams c;
    c.s0 = buf_load4f(rs, 0);
    c.s1 = buf_load4f(rs, 4);
    c.s2 = buf_load4f(rs, 8);
    c.b_e = buf_load4f(rb, (uint32_t)e * 4);
    c.b_8e = buf_load4f(rb, (uint32_t)(8 + e) * 4);
    return c;
}

// The coefficients of token t from its reduced partial row: lane e of a 16-lane
// group holds entries e (a0) and 16 + e (a1). Every lane of the wave must call it
// (row and column sums are DPP steps within the group); only lanes with `store`
// write.
__device__ __forceinline__ void finalize_coeffs(const FinalizeArgs& f, const CoefParams& cp, int64_t t, int e,
                                                float a0, float a1, bool store) {
    // No contraction: the compiler would fuse a lane's own product into the first
    // add of a column sum while the partner's term arrives rounded, so the four
    // lanes of a comb column would not add the same numbers; the fused
    // multiply-adds meant here are written out.
#pragma clang fp contract(off)
    const int lane16 = (threadIdx.x & 63) & ~15;
    const float sumsq = __shfl(a1, lane16 + (kMix - 16));
    const float rstd = 1.0f / sqrtf(sumsq / (float)f.D + f.norm_eps);
    const float m0 = a0 * rstd;            // mixes[e]
    const float m1 = a1 * rstd;            // mixes[16 + e] (valid for e < 8)
    if (f.mixes && store) {
        f.mixes[t * kMix + e] = m0;
        if (e < kMix - 16) f.mixes[t * kMix + 16 + e] = m1;
    }
    if (!f.split) return;                  // uniform
    // comb logit of entry e is mixes[8 + e]: lane 8+e's m0 for e < 8, lane e-8's m1 otherwise
    const float lo = __shfl(m0, lane16 + ((8 + e) & 15));
    const float hi = __shfl(m1, lane16 + ((e + 8) & 15));
    const float m = e < 8 ? lo : hi;
    float c = fmaf(m, cp.s2, cp.b_8e);
    // row softmax (max subtracted), + eps
    float mx = fmaxf(c, dpp<kQuadSwap1>(c));
    mx = fmaxf(mx, dpp<kQuadSwap2>(mx));
    c = __expf(c - mx);
    c = fmaf(c, __builtin_amdgcn_rcpf(row_sum16(c)), f.eps);
    c *= __builtin_amdgcn_rcpf(col_sum16(c) + f.eps);
    for (int it = 1; it < f.iters; ++it) {
        c *= __builtin_amdgcn_rcpf(row_sum16(c) + f.eps);
        c *= __builtin_amdgcn_rcpf(col_sum16(c) + f.eps);
    }
    if (store) {
        f.comb[t * 16 + e] = c;
        if (e < kHC) f.pre[t * kHC + e] = sigmoid(fmaf(m0, cp.s0, cp.b_e)) + f.eps;
        else if (e < 2 * kHC) f.post[t * kHC + e - kHC] = 2.0f * sigmoid(fmaf(m0, cp.s1, cp.b_e));
    }
}

// 16 lanes per token: token t (shared by the 16-lane group; t >= n: computes on
// token 0, stores nothing), lane e of the group reduces entries e and 16 + e over
// the slices in order. Serves up to kFin16Slices slices (more take the wave
// finalize): every slice's load is issued before the first wait; slices past
// nsplit re-read the last one and are weighted by zero (v * 0 = 0, v * 1 = v, so
// the sum is that of the real slices, in order).
constexpr int kFin16Slices = 8;

__device__ __forceinline__ void finalize16(const FinalizeArgs& f, int64_t t, int e) {
    const bool ok = t < f.n;
    const int64_t tt = ok ? t : 0;
    const CoefParams cp = load_coef_params(f, e);
    float v0[kFin16Slices], v1[kFin16Slices];
#pragma unroll
    for (int s = 0; s < kFin16Slices; ++s) {
        const int sc = s < f.nsplit ? s : f.nsplit - 1;
        const float* p = f.part + ((int64_t)sc * f.n + tt) * kPart;
        v0[s] = p[e];
        v1[s] = p[16 + e];                 // entries 16..31; 25..31 are never used below
    }
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int s = 0; s < kFin16Slices; ++s) {
        const float m = s < f.nsplit ? 1.f : 0.f;
        a0 += v0[s] * m;
        a1 += v1[s] * m;
    }
    finalize_coeffs(f, cp, t, e, a0, a1, ok);
}

constexpr int kFinBlock = 256;

__global__ __launch_bounds__(kFinBlock) void finalize_kernel(FinalizeArgs f) {
    pin_args(f);
    finalize16(f, ((int64_t)blockIdx.x * kFinBlock + threadIdx.x) >> 4, threadIdx.x & 15);
}

// A wave per token, for many slices: lane l reads float4 l % 8 (entries
// 4 (l % 8) .. + 3) of slices l / 8, l / 8 + 8, ...; every load is issued before
// the first wait, and slices past nsplit read as zero (masked offsets). The 8
// slice groups are then summed by an xor tree in a fixed order (lane l + lane
// l ^ 8 by a row rotation, then l ^ 16 and l ^ 32 by gfx950's lane swaps), and
// each 16-lane group takes entries e and 16 + e from the 32 sums, passed through
// the wave's own LDS row, for the coefficient step (all four groups hold the same
// token; the first stores).
constexpr int kFinWaveRounds = 16;   // slices per lane: nsplit <= 128

// v + the value of lane l ^ kSpan (kSpan = 16 or 32): gfx950's lane swaps with
// both operands v return v and its partner, one in each result.
template <int kSpan>
__device__ __forceinline__ float add_partner(float v) {
    const uint32_t u = __float_as_uint(v);
    if constexpr (kSpan == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

__global__ __launch_bounds__(kFinBlock) void finalize_wave_kernel(FinalizeArgs f) {
    __shared__ float4 sums[kFinBlock / 64][8];
    pin_args(f);
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * (kFinBlock / 64) + uniform(threadIdx.x >> 6);
    const bool ok = t < f.n;
    const int64_t tt = ok ? t : 0;
    const int g = lane >> 3, q = lane & 7;
    const CoefParams cp = load_coef_params(f, lane & 15);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(f.part, (int64_t)f.nsplit * f.n * kPart * (int64_t)sizeof(float));
    // the rounds the slice count needs (uniform); the loads of the others are skipped
    const int rounds = (f.nsplit + 7) / 8;
    float4 v[kFinWaveRounds];
#pragma unroll
    for (int k = 0; k < kFinWaveRounds; ++k) {
        v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (k < rounds) {
            const int64_t s = g + 8 * k;
            const uint32_t off =
                s < f.nsplit ? (uint32_t)(((s * f.n + tt) * kPart + 4 * q) * sizeof(float)) : kOffMasked;
            v[k] = buf_load16f(r, off, 0);
        }
    }
    float4 acc = v[0];
#pragma unroll
    for (int k = 1; k < kFinWaveRounds; ++k) {
        acc.x += v[k].x; acc.y += v[k].y; acc.z += v[k].z; acc.w += v[k].w;
    }
    acc.x += dpp<kRowRor8>(acc.x); acc.y += dpp<kRowRor8>(acc.y);
    acc.z += dpp<kRowRor8>(acc.z); acc.w += dpp<kRowRor8>(acc.w);
    acc.x = add_partner<16>(acc.x); acc.y = add_partner<16>(acc.y);
    acc.z = add_partner<16>(acc.z); acc.w = add_partner<16>(acc.w);
    acc.x = add_partner<32>(acc.x); acc.y = add_partner<32>(acc.y);
    acc.z = add_partner<32>(acc.z); acc.w = add_partner<32>(acc.w);
    // lanes 0..7 hold entries 4 l .. 4 l + 3 of the sum; the LDS operations of one
    // wave complete in order, so its reads below see its writes
    float4* row = sums[threadIdx.x >> 6];
    if (lane < 8) row[lane] = acc;
    const int e = lane & 15;
    const float a0 = reinterpret_cast<const float*>(row)[e];
    const float a1 = reinterpret_cast<const float*>(row)[16 + e];
    finalize_coeffs(f, cp, t, e, a0, a1, ok && lane < 16);
}

// ------------------------------------------------- bf16 projection weights
// The 24 mix columns take 5 B operands per 32-channel k-block and stream:
// hi, mid, lo of mixes 0..15 (one accumulator), then [hi | mid] and [lo | 0] of
// mixes 16..23 (a second accumulator whose two 8-column halves are added at the
// end).
constexpr int kFragsPerKb = 5;

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

// ------------------------------------------------ bf16 sweep: shared pieces
// The bf16 sweep walks a channel slice in steps of 64 channels (two 32-channel
// k-blocks). In its rowwise role lane (t8 = lane/8, c8 = lane%8) of wave w owns
// token 8w + t8 and channels cs + 8*c8 .. +8 of step cs, in all 4 streams and in
// the sublayer output: one 16-byte load per stream, one instruction = 8 tokens x
// 128 B. Expanded / collapsed values are written, XOR-swizzled, into an LDS A
// region from which the MFMA role reads 16-token x 32-channel operands.
constexpr int kStep = 64;                                  // channels per step
constexpr int kStepKb = kStep / kChunk;                     // k-blocks per step


// A slot of (token t, stream j, 8-channel group q): rows (t, j) of 128 B; the
// stream index is XORed with t's parity and the group with (t/2) % 8, so that an
// MFMA A read (16 consecutive tokens at one group) and a rowwise write (2 tokens
// x 8 groups per 16 lanes) each cover the 16 bank groups of a 256-byte window.
__device__ __forceinline__ int a_slot(int t, int j, int q) {
    return ((t * kHC + (j ^ (t & 1))) << 3) + (q ^ ((t >> 1) & 7));
}

template <bool kPost>
struct StepRegs {
    uint4 x[kHC];   // 8 channels of each stream
    uint4 f;        // 8 channels of the sublayer output (expand only)
};

// ------------------------------------------------------------ bf16 sweep
// Workgroup = 8 waves x 8 tokens = 64 tokens (four 16-token MFMA row tiles) x one
// channel slice, walked in steps of 64 channels (two 32-channel k-blocks); one
// workgroup per CU.
//   - rowwise role (see above); the stream loads run two steps ahead in three
//     register sets.
//   - MFMA role: wave w multiplies stream j = w % 4 for k-block w / 4 of the step
//     across all four row tiles, so every weight fetched from L2 serves 64
//     tokens. Its fp32 weights (8 channels of two mix rows per lane, 64 B) are
//     double-buffered and issued one step ahead, before that step's stream
//     loads: vmcnt retires in issue order, so waiting for the weights only waits
//     for loads at least two steps old. After the barrier they are split into
//     three bf16 terms (hi + mid + lo, ~24 significant bits) that form the 5 B
//     operands; the split's VALU work hides under the memory-bound step.
//   - the step loop is unrolled by six (three stream sets x two weight sets) so
//     every set keeps fixed registers.
constexpr int kSwWaves = 8;
constexpr int kSwBlock = kSwWaves * 64;
constexpr int kSwTok = 64;
constexpr int kSwASlots = kSwTok * kHC * (kStep / 8);     // 16-byte slots per A buffer (32 KB)
constexpr int kSweepTargetGroups = 256;   // one workgroup per CU
// From this many tokens on the bf16 sweep takes 128-token groups (bf16_sweep2_kernel);
// below it, 128-token groups would leave lanes idle (decode: 64 tokens).
constexpr int64_t kWideSweepTokens = 1024;

struct SweepLds {
    uint4 a[2][kSwASlots];                 // 64 KB; reused for the cross-wave reduction
    float ss[kSwWaves][4][16];             // Gram diagonals per wave and tile
};

// The cross-wave sum of the MFMA accumulators, after every wave has written its
// own to red[wave][T][nt][lane] (kT 16-token row tiles, 2 mix tiles): thread
// (T, nt, l) adds the 8 waves' float4s in wave order and stores its 4 tokens'
// dots (accumulator entry ii of lane l is token 16 T + 4 (l / 16) + ii, mix
// 16 nt + l % 16).
template <int kT>
__device__ __forceinline__ void red_store(const floatx4_t* red, float* __restrict__ part, int64_t tok0, int64_t n) {
#pragma unroll
    for (int e = threadIdx.x; e < kT * 2 * 64; e += kSwBlock) {
        const int l = e & 63, nt = (e >> 6) & 1, T = e >> 7;
        floatx4_t sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kSwWaves; ++w) sum += red[w * kT * 2 * 64 + e];
        const int mix = nt * 16 + (l & 15);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int64_t t = tok0 + T * 16 + 4 * (l >> 4) + ii;
            if (mix < kMix && t < n) part[t * kPart + mix] = sum[ii];
        }
    }
}

// kOne: every slice is a single step (decode: 64 tokens, 80 slices of 64
// channels); no loads are issued ahead, since they would all be masked and at
// this size every wave instruction is on the critical path.
template <bool kPost, bool kPre, bool kOne>
__global__ __launch_bounds__(kSwBlock) void bf16_sweep_kernel(PassArgs a) {
    __shared__ SweepLds lds;
    pin_args(a);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int mj = wave & 3, mkk = wave >> 2;    // MFMA role: stream, k-block of the step
    const int t8 = lane >> 3, c8 = lane & 7;     // rowwise role
    const int64_t n = a.n, d = a.d;
    const int nkb = a.nchunks;
    const int split = (int)(blockIdx.x % (unsigned)a.nsplit);
    const int64_t group = blockIdx.x / (unsigned)a.nsplit;
    const int64_t tok0 = group * kSwTok;
    const int tl = wave * 8 + t8;
    const bool tok_ok = tok0 + tl < n;
    const int kb_begin = split * a.chunks_per_split;
    const int kb_end = min(nkb, kb_begin + a.chunks_per_split);
    const int64_t c_begin = (int64_t)kb_begin * kChunk;
    const int64_t c_end = min(d, (int64_t)kb_end * kChunk);
    const int nst = (int)((c_end - c_begin + kStep - 1) / kStep);   // >= 1: slices are never empty

    // The token's coefficients, as raw buffer loads (a token past n reads zeros):
    // no branch, so nothing waits for them before the rowwise work uses them. A
    // guarded load inside a branch made the compiler wait for it at the branch's
    // end, a memory round trip before the first stream load was issued.
    float pk[kHC], cm[kHC * kHC], pim[kHC];
#pragma unroll
    for (int i = 0; i < kHC; ++i) pk[i] = pim[i] = 0.f;
#pragma unroll
    for (int i = 0; i < kHC * kHC; ++i) cm[i] = 0.f;
    const uint32_t lane_c = tok_ok ? (uint32_t)(tl * 16) : kOffMasked;   // 16 B per token and row of 4
    if constexpr (kPost) {
        const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.post_prev + tok0 * kHC, (n - tok0) * 16);
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.comb_prev + tok0 * kHC * kHC, (n - tok0) * 64);
        const uint32_t lane_cc = tok_ok ? (uint32_t)(tl * 64) : kOffMasked;
        const float4 pv = buf_load16f(rp, lane_c, 0);
        pk[0] = pv.x; pk[1] = pv.y; pk[2] = pv.z; pk[3] = pv.w;
#pragma unroll
        for (int j = 0; j < kHC; ++j) {
            const float4 cv = buf_load16f(rc, lane_cc, (uint32_t)(j * 16));
            cm[4 * j] = cv.x; cm[4 * j + 1] = cv.y; cm[4 * j + 2] = cv.z; cm[4 * j + 3] = cv.w;
        }
    }
    if constexpr (kPre) {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.pre_mix + tok0 * kHC, (n - tok0) * 16);
        const float4 pv = buf_load16f(rq, lane_c, 0);
        pim[0] = pv.x; pim[1] = pv.y; pim[2] = pv.z; pim[3] = pv.w;
    }

    const int64_t row_x = kHC * d * 2, row_f = d * 2;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const char*>(a.res) + tok0 * row_x, (n - tok0) * row_x);
    const __amdgpu_buffer_rsrc_t rf = make_rsrc(kPost ? static_cast<const char*>(a.f) + tok0 * row_f : nullptr,
                                                kPost ? (n - tok0) * row_f : 0);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(kPost ? static_cast<char*>(a.streams_out) + tok0 * row_x : nullptr,
                                                kPost ? (n - tok0) * row_x : 0);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(kPre ? static_cast<char*>(a.y) + tok0 * row_f : nullptr,
                                                kPre ? (n - tok0) * row_f : 0);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.hc_fn, (int64_t)kMix * kHC * d * 4);
    const uint32_t lane_x = tok_ok ? (uint32_t)(tl * row_x + c8 * 16) : kOffMasked;
    const uint32_t lane_f = tok_ok ? (uint32_t)(tl * row_f + c8 * 16) : kOffMasked;
    // MFMA role, B operand lane (k-group g = lane/16, column col = lane%16): fp32
    // weights of mix row col (column tile 0) and 16 + col%8 (tile 1), channels
    // 8g .. 8g+7 of stream mj's k-block
    const int g = lane >> 4, col = lane & 15;
    const uint32_t lane_w0 = (uint32_t)(((int64_t)col * kHC * d + (int64_t)mj * d + g * 8) * 4);
    const uint32_t lane_w1 = (uint32_t)(((int64_t)(16 + (col & 7)) * kHC * d + (int64_t)mj * d + g * 8) * 4);

    auto load_step = [&](StepRegs<kPost>& R, int s) {
        const int64_t cs = c_begin + (int64_t)s * kStep;
        const bool ok = cs + c8 * 8 < c_end;
        const uint32_t vx = ok ? lane_x : kOffMasked, vf = ok ? lane_f : kOffMasked;
        const uint32_t so = (uint32_t)(cs * 2);
#pragma unroll
        for (int j = 0; j < kHC; ++j) R.x[j] = buf_load16(rx, vx, so + (uint32_t)(j * row_f));
        if constexpr (kPost) R.f = buf_load16(rf, vf, so);
    };
    // fp32 weights of (stream mj, k-block mkk of step s): 8 channels of two mix
    // rows per lane; past the slice or past d: zeros
    auto load_b = [&](float4 (&W)[4], int s) {
        const int kb = kb_begin + s * kStepKb + mkk;
        const bool ok = kb < kb_end && (int64_t)kb * kChunk + g * 8 < d;   // d % 8 == 0: whole groups
        const uint32_t v0 = ok ? lane_w0 : kOffMasked, v1 = ok ? lane_w1 : kOffMasked;
        const uint32_t so = (uint32_t)(kb * kChunk * 4);
        W[0] = buf_load16f(rw, v0, so);
        W[1] = buf_load16f(rw, v0 + 16u, so);
        W[2] = buf_load16f(rw, v1, so);
        W[3] = buf_load16f(rw, v1 + 16u, so);
    };

    floatx4_t acc[4][2], gram[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) acc[T][0] = acc[T][1] = gram[T] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    auto step = [&](int s, StepRegs<kPost>& cur, StepRegs<kPost>& ahead, float4 (&Wcur)[4], float4 (&Wnext)[4],
                    bool prefetch = true) {
        if (prefetch) {
            load_b(Wnext, s + 1);
            load_step(ahead, s + 2);
        }
        const int64_t cs = c_begin + (int64_t)s * kStep;
        const bool ok = cs + c8 * 8 < c_end;
        const uint32_t vx = ok ? lane_x : kOffMasked, vf = ok ? lane_f : kOffMasked;
        const uint32_t so = (uint32_t)(cs * 2);
        uint32_t yw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t xw[kHC];
#pragma unroll
            for (int j = 0; j < kHC; ++j) xw[j] = (&cur.x[j].x)[w];
            if constexpr (kPost) {
                const uint32_t fw = (&cur.f.x)[w];
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
                for (int k = 0; k < kHC; ++k) xw[k] = (&cur.x[k].x)[w] = ow[k];
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
            for (int k = 0; k < kHC; ++k) buf_store16(cur.x[k], ro, vx, so + (uint32_t)(k * row_f));
        }
        if constexpr (kPre) buf_store16(make_uint4(yw[0], yw[1], yw[2], yw[3]), ry, vf, so);
        uint4* A = lds.a[s & 1];
#pragma unroll
        for (int j = 0; j < kHC; ++j) A[a_slot(tl, j, c8)] = cur.x[j];
        __syncthreads();   // A buffer complete; the other buffer is free again
        // B operands: weights split into three bf16 terms (hi + mid + lo); column
        // tile 1 packs [hi | mid] and [lo | 0] of mixes 16..23 into two operands
        uint4 Bcur[kFragsPerKb], hi1, mid1, lo1;
        split3(Wcur[0], Wcur[1], Bcur[0], Bcur[1], Bcur[2]);
        split3(Wcur[2], Wcur[3], hi1, mid1, lo1);
        const bool lo_half = col < 8;
        Bcur[3] = make_uint4(lo_half ? hi1.x : mid1.x, lo_half ? hi1.y : mid1.y, lo_half ? hi1.z : mid1.z,
                             lo_half ? hi1.w : mid1.w);
        Bcur[4] = make_uint4(lo_half ? lo1.x : 0u, lo_half ? lo1.y : 0u, lo_half ? lo1.z : 0u, lo_half ? lo1.w : 0u);
        // the four A reads are issued before the first MFMA (a scheduling barrier
        // keeps them there): otherwise each read's latency sits between two MFMA
        // groups
        bf16x8_t Av[4];
#pragma unroll
        for (int T = 0; T < 4; ++T)
            Av[T] = __builtin_bit_cast(bf16x8_t, A[a_slot(T * 16 + (lane & 15), mj, mkk * 4 + (lane >> 4))]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int T = 0; T < 4; ++T) {
#pragma unroll
            for (int q = 0; q < kFragsPerKb; ++q)
                acc[T][q < 3 ? 0 : 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    Av[T], __builtin_bit_cast(bf16x8_t, Bcur[q]), acc[T][q < 3 ? 0 : 1], 0, 0, 0);
            gram[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Av[T], Av[T], gram[T], 0, 0, 0);
        }
    };

    StepRegs<kPost> R0, R1, R2;
    float4 B0[4], B1[4];
    load_b(B0, 0);
    load_step(R0, 0);
    if constexpr (kOne) {
        step(0, R0, R2, B0, B1, false);
    } else {
        load_step(R1, 1);
        // Whole groups of six steps in a loop without exits, the remaining steps
        // after it: the loads pending at the loop head are then the same on every
        // path into it, and the compiler need not drain them there.
        int s = 0;
        for (; s + 6 <= nst; s += 6) {
            step(s, R0, R2, B0, B1);
            step(s + 1, R1, R0, B1, B0);
            step(s + 2, R2, R1, B0, B1);
            step(s + 3, R0, R2, B1, B0);
            step(s + 4, R1, R0, B0, B1);
            step(s + 5, R2, R1, B1, B0);
        }
        if (s < nst) step(s, R0, R2, B0, B1);
        if (s + 1 < nst) step(s + 1, R1, R0, B1, B0);
        if (s + 2 < nst) step(s + 2, R2, R1, B0, B1);
        if (s + 3 < nst) step(s + 3, R0, R2, B1, B0);
        if (s + 4 < nst) step(s + 4, R1, R0, B0, B1);
    }

    __syncthreads();   // every wave is done with the A buffers
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) acc[T][1][ii] += dpp<kRowRor8>(acc[T][1][ii]);
    floatx4_t* red = reinterpret_cast<floatx4_t*>(&lds.a[0][0]);   // [wave][T][nt][lane], 64 KB
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) red[((wave * 4 + T) * 2 + nt) * 64 + lane] = acc[T][nt];
    // Gram diagonal: lane (g, col) holds entry (4 g + ii, col) of each row tile's
    // A A^T, so at most one diagonal entry per tile, ii = col - 4 g; one
    // predicated store per tile (a branch per candidate entry cost more)
    const int dii = col - 4 * g;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
        const float v = dii == 0 ? gram[T][0] : dii == 1 ? gram[T][1] : dii == 2 ? gram[T][2] : gram[T][3];
        if ((unsigned)dii < 4u) lds.ss[wave][T][col] = v;
    }
    __syncthreads();
    float* part = a.part + (int64_t)split * n * kPart;
    red_store<4>(red, part, tok0, n);
    if (threadIdx.x < kSwTok) {   // token T*16 + row of the group
        const int T = threadIdx.x >> 4, row = threadIdx.x & 15;
        const int64_t t = tok0 + threadIdx.x;
        if (t < n) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < kSwWaves; ++w) s += lds.ss[w][T][row];
            part[t * kPart + kMix] = s;
        }
    }
}

// ------------------------------------------------ bf16 sweep, 128-token groups
// The same data flow as bf16_sweep_kernel with 128 tokens per workgroup, so that
// every weight fetched from L2 serves 128 tokens (half the L2 weight traffic per
// token); used from kWideSweepTokens tokens on. Lane (t8, c8) of wave w owns
// tokens 8w + t8 and 64 + 8w + t8 (8 channels per step each). To fit the
// registers: the per-token coefficients stay in LDS, the streams are prefetched
// one step ahead (one step of 128 tokens: the same bytes in flight as two steps
// of 64), and the sum of squares is taken on the VALU from the (rounded) stream
// values, summed over a token row's 8 lanes in a fixed order, instead of an MFMA
// Gram diagonal.
constexpr int kS2Tok = 2 * kSwTok;
constexpr int kS2ASlots = kS2Tok * kHC * (kStep / 8);     // 64 KB per A buffer
constexpr int kS2Coef = 6;                                // float4: post, comb rows 0..3, pre_mix

struct Sweep2Lds {
    uint4 a[2][kS2ASlots];                 // 128 KB; reused for the cross-wave reduction
    float4 coef[kS2Tok][kS2Coef];          // 12 KB
};

template <bool kPost>
struct StepRegs2 {
    uint4 x[2][kHC];
    uint4 f[2];
};

template <bool kPost, bool kPre>
__global__ __launch_bounds__(kSwBlock) void bf16_sweep2_kernel(PassArgs a) {
    __shared__ Sweep2Lds lds;
    pin_args(a);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int mj = wave & 3, mkk = wave >> 2;
    const int t8 = lane >> 3, c8 = lane & 7;
    const int64_t n = a.n, d = a.d;
    const int nkb = a.nchunks;
    const int split = (int)(blockIdx.x % (unsigned)a.nsplit);
    const int64_t group = blockIdx.x / (unsigned)a.nsplit;
    const int64_t tok0 = group * kS2Tok;
    const int tlh[2] = {wave * 8 + t8, kSwTok + wave * 8 + t8};
    const int kb_begin = split * a.chunks_per_split;
    const int kb_end = min(nkb, kb_begin + a.chunks_per_split);
    const int64_t c_begin = (int64_t)kb_begin * kChunk;
    const int64_t c_end = min(d, (int64_t)kb_end * kChunk);
    const int nst = (int)((c_end - c_begin + kStep - 1) / kStep);

    const int64_t row_x = kHC * d * 2, row_f = d * 2;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const char*>(a.res) + tok0 * row_x, (n - tok0) * row_x);
    const __amdgpu_buffer_rsrc_t rf = make_rsrc(kPost ? static_cast<const char*>(a.f) + tok0 * row_f : nullptr,
                                                kPost ? (n - tok0) * row_f : 0);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(kPost ? static_cast<char*>(a.streams_out) + tok0 * row_x : nullptr,
                                                kPost ? (n - tok0) * row_x : 0);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(kPre ? static_cast<char*>(a.y) + tok0 * row_f : nullptr,
                                                kPre ? (n - tok0) * row_f : 0);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.hc_fn, (int64_t)kMix * kHC * d * 4);
    uint32_t lane_x[2], lane_f[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const bool ok = tok0 + tlh[h] < n;
        lane_x[h] = ok ? (uint32_t)(tlh[h] * row_x + c8 * 16) : kOffMasked;
        lane_f[h] = ok ? (uint32_t)(tlh[h] * row_f + c8 * 16) : kOffMasked;
    }
    const int g = lane >> 4, col = lane & 15;
    const uint32_t lane_w0 = (uint32_t)(((int64_t)col * kHC * d + (int64_t)mj * d + g * 8) * 4);
    const uint32_t lane_w1 = (uint32_t)(((int64_t)(16 + (col & 7)) * kHC * d + (int64_t)mj * d + g * 8) * 4);

    auto load_step = [&](StepRegs2<kPost>& R, int s) {
        const int64_t cs = c_begin + (int64_t)s * kStep;
        const bool ok = cs + c8 * 8 < c_end;
        const uint32_t so = (uint32_t)(cs * 2);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t vx = ok ? lane_x[h] : kOffMasked, vf = ok ? lane_f[h] : kOffMasked;
#pragma unroll
            for (int j = 0; j < kHC; ++j) R.x[h][j] = buf_load16(rx, vx, so + (uint32_t)(j * row_f));
            if constexpr (kPost) R.f[h] = buf_load16(rf, vf, so);
        }
    };
    auto load_b = [&](float4 (&W)[4], int s) {
        const int kb = kb_begin + s * kStepKb + mkk;
        const bool ok = kb < kb_end && (int64_t)kb * kChunk + g * 8 < d;
        const uint32_t v0 = ok ? lane_w0 : kOffMasked, v1 = ok ? lane_w1 : kOffMasked;
        const uint32_t so = (uint32_t)(kb * kChunk * 4);
        W[0] = buf_load16f(rw, v0, so);
        W[1] = buf_load16f(rw, v0 + 16u, so);
        W[2] = buf_load16f(rw, v1, so);
        W[3] = buf_load16f(rw, v1 + 16u, so);
    };

    floatx4_t acc[8][2];
#pragma unroll
    for (int T = 0; T < 8; ++T) acc[T][0] = acc[T][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    float ssq[2] = {0.f, 0.f};

    // Stream prefetch: with the expand, the set just consumed takes step s + 2 right
    // after the rowwise work of step s, before the barrier and the MFMAs; without
    // it, step s + 1 is issued into the other set at the start of step s (measured:
    // each order is the faster one for its instance).
    auto step = [&](int s, StepRegs2<kPost>& cur, StepRegs2<kPost>& ahead, float4 (&Wcur)[4],
                    float4 (&Wnext)[4]) {
        load_b(Wnext, s + 1);
        if constexpr (!kPost) load_step(ahead, s + 1);
        const int64_t cs = c_begin + (int64_t)s * kStep;
        const bool ok = cs + c8 * 8 < c_end;
        const uint32_t so = (uint32_t)(cs * 2);
        uint4* A = lds.a[s & 1];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int tl = tlh[h];
            const uint32_t vx = ok ? lane_x[h] : kOffMasked, vf = ok ? lane_f[h] : kOffMasked;
            float pk[kHC], cm[kHC * kHC], pim[kHC];
            if constexpr (kPost) {
                const float4 pv = lds.coef[tl][0];
                pk[0] = pv.x; pk[1] = pv.y; pk[2] = pv.z; pk[3] = pv.w;
#pragma unroll
                for (int j = 0; j < kHC; ++j) {
                    const float4 cv = lds.coef[tl][1 + j];
                    cm[4 * j] = cv.x; cm[4 * j + 1] = cv.y; cm[4 * j + 2] = cv.z; cm[4 * j + 3] = cv.w;
                }
            }
            if constexpr (kPre) {
                const float4 pv = lds.coef[tl][5];
                pim[0] = pv.x; pim[1] = pv.y; pim[2] = pv.z; pim[3] = pv.w;
            }
            uint32_t yw[4];
            float sq = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t xw[kHC];
#pragma unroll
                for (int j = 0; j < kHC; ++j) xw[j] = (&cur.x[h][j].x)[w];
                if constexpr (kPost) {
                    const uint32_t fw = (&cur.f[h].x)[w];
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
                    for (int k = 0; k < kHC; ++k) xw[k] = (&cur.x[h][k].x)[w] = ow[k];
                }
                float y0 = 0.f, y1 = 0.f;
#pragma unroll
                for (int j = 0; j < kHC; ++j) {
                    const float a0 = bf16_lo(xw[j]), a1 = bf16_hi(xw[j]);
                    sq = fmaf(a0, a0, sq);
                    sq = fmaf(a1, a1, sq);
                    if constexpr (kPre) {
                        y0 = fmaf(pim[j], a0, y0);
                        y1 = fmaf(pim[j], a1, y1);
                    }
                }
                if constexpr (kPre) yw[w] = pack_bf16x2(y0, y1);
            }
            ssq[h] += sq;
            if constexpr (kPost) {
#pragma unroll
                for (int k = 0; k < kHC; ++k) buf_store16(cur.x[h][k], ro, vx, so + (uint32_t)(k * row_f));
            }
            if constexpr (kPre) buf_store16(make_uint4(yw[0], yw[1], yw[2], yw[3]), ry, vf, so);
#pragma unroll
            for (int j = 0; j < kHC; ++j) A[a_slot(tl, j, c8)] = cur.x[h][j];
        }
        if constexpr (kPost) load_step(cur, s + 2);
        __syncthreads();
        uint4 Bcur[kFragsPerKb], hi1, mid1, lo1;
        split3(Wcur[0], Wcur[1], Bcur[0], Bcur[1], Bcur[2]);
        split3(Wcur[2], Wcur[3], hi1, mid1, lo1);
        const bool lo_half = col < 8;
        Bcur[3] = make_uint4(lo_half ? hi1.x : mid1.x, lo_half ? hi1.y : mid1.y, lo_half ? hi1.z : mid1.z,
                             lo_half ? hi1.w : mid1.w);
        Bcur[4] = make_uint4(lo_half ? lo1.x : 0u, lo_half ? lo1.y : 0u, lo_half ? lo1.z : 0u, lo_half ? lo1.w : 0u);
        // Without the expand, each A read is issued one row tile ahead of its MFMAs
        // (a scheduling barrier keeps it there), so its latency overlaps the
        // previous tile's MFMAs; the expand instance has no registers to spare for it.
        if constexpr (kPost) {
#pragma unroll
            for (int T = 0; T < 8; ++T) {
                const bf16x8_t Av =
                    __builtin_bit_cast(bf16x8_t, A[a_slot(T * 16 + (lane & 15), mj, mkk * 4 + (lane >> 4))]);
#pragma unroll
                for (int q = 0; q < kFragsPerKb; ++q)
                    acc[T][q < 3 ? 0 : 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        Av, __builtin_bit_cast(bf16x8_t, Bcur[q]), acc[T][q < 3 ? 0 : 1], 0, 0, 0);
            }
        } else {
            auto read_a = [&](int T) {
                return __builtin_bit_cast(bf16x8_t, A[a_slot(T * 16 + (lane & 15), mj, mkk * 4 + (lane >> 4))]);
            };
            bf16x8_t Acur = read_a(0);
#pragma unroll
            for (int T = 0; T < 8; ++T) {
                bf16x8_t Anext = Acur;
                if (T + 1 < 8) Anext = read_a(T + 1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = 0; q < kFragsPerKb; ++q)
                    acc[T][q < 3 ? 0 : 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        Acur, __builtin_bit_cast(bf16x8_t, Bcur[q]), acc[T][q < 3 ? 0 : 1], 0, 0, 0);
                Acur = Anext;
            }
        }
    };

    // The per-token coefficients go to LDS, loaded with the first step's loads
    // and written after those are issued (a load behind a branch, written at
    // once, would make every wave wait a memory round trip before its first
    // stream load). Item i of the list [post (128) | comb rows (4 x 128) | pre_mix
    // (128)], as far as the instance uses them, is thread i % 512's load r = i /
    // 512; each wave's 64 items come from one array, so the source is uniform.
    // Tokens past n read as zeros (the buffer ranges end at n).
    constexpr int kNPost = kPost ? kS2Tok : 0, kNComb = kPost ? kS2Tok * kHC : 0, kNPre = kPre ? kS2Tok : 0;
    constexpr int kNCoef = kNPost + kNComb + kNPre;
    constexpr int kCoefLoads = (kNCoef + kSwBlock - 1) / kSwBlock;
    const __amdgpu_buffer_rsrc_t rcp = make_rsrc(kPost ? a.post_prev + tok0 * kHC : nullptr, kPost ? (n - tok0) * 16 : 0);
    const __amdgpu_buffer_rsrc_t rcc =
        make_rsrc(kPost ? a.comb_prev + tok0 * kHC * kHC : nullptr, kPost ? (n - tok0) * 64 : 0);
    const __amdgpu_buffer_rsrc_t rcq = make_rsrc(kPre ? a.pre_mix + tok0 * kHC : nullptr, kPre ? (n - tok0) * 16 : 0);
    float4 coef_v[kCoefLoads > 0 ? kCoefLoads : 1];
    auto coef_item = [&](int r, int& first, int& j, int& seg) {   // seg 0 post, 1 comb, 2 pre_mix
        first = uniform((uint32_t)(r * kSwBlock + wave * 64));
        const int i = r * kSwBlock + (int)threadIdx.x;
        seg = first < kNPost ? 0 : first < kNPost + kNComb ? 1 : 2;
        j = i - (seg == 0 ? 0 : seg == 1 ? kNPost : kNPost + kNComb);
    };
#pragma unroll
    for (int r = 0; r < kCoefLoads; ++r) {
        int first, j, seg;
        coef_item(r, first, j, seg);
        if (first < kNCoef) coef_v[r] = buf_load16f(seg == 0 ? rcp : seg == 1 ? rcc : rcq, (uint32_t)j * 16, 0);
    }
    StepRegs2<kPost> R0, R1;
    float4 B0[4], B1[4];
    load_b(B0, 0);
    load_step(R0, 0);
    if constexpr (kPost) load_step(R1, 1);
#pragma unroll
    for (int r = 0; r < kCoefLoads; ++r) {
        int first, j, seg;
        coef_item(r, first, j, seg);
        if (first < kNCoef) {
            if (seg == 0) lds.coef[j][0] = coef_v[r];
            else if (seg == 1) lds.coef[j >> 2][1 + (j & 3)] = coef_v[r];
            else lds.coef[j][5] = coef_v[r];
        }
    }
    __syncthreads();   // the coefficients are in LDS
    int s = 0;
    for (; s + 2 <= nst; s += 2) {
        step(s, R0, R1, B0, B1);
        step(s + 1, R1, R0, B1, B0);
    }
    if (s < nst) step(s, R0, R1, B0, B1);

    __syncthreads();   // every wave is done with the A buffers
#pragma unroll
    for (int T = 0; T < 8; ++T)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) acc[T][1][ii] += dpp<kRowRor8>(acc[T][1][ii]);
    floatx4_t* red = reinterpret_cast<floatx4_t*>(&lds.a[0][0]);   // [wave][T][nt][lane], 128 KB
#pragma unroll
    for (int T = 0; T < 8; ++T)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) red[((wave * 8 + T) * 2 + nt) * 64 + lane] = acc[T][nt];
    float* part = a.part + (int64_t)split * n * kPart;
    // sum of squares: the 8 lanes of a token row (xor 1, 2, 4), in a fixed order
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float v = ssq[h];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        const int64_t t = tok0 + tlh[h];
        if (c8 == 0 && t < n) part[t * kPart + kMix] = v;
    }
    __syncthreads();
    red_store<8>(red, part, tok0, n);
}

// ------------------------------------------- sublayer RMSNorm + MXFP8 cast
// The sublayer input after the collapse is RMS-normalised with a learned gain
// (Block.forward: attn_norm / ffn_norm) and cast to MXFP8 for the projections
// that read it (diagram "Cast to MXFP8"). Pass 1 sums the squares of a row;
// pass 2 multiplies by 1/sqrt(mean + eps) and the gain, rounds to the row dtype
// (the normalised output), and casts groups of 32 channels: four consecutive
// lanes own a group (8 channels each), its amax is combined with two quad DPP
// steps.
constexpr int kNormBlock = 256;

// ceil(log2(max(a, 1e-4) / 448)) for a >= 0, exactly: 448 = 1.75 * 2^8, so for
// a = m * 2^e (m in [1, 2)) the exponent is e - 8, plus one when m > 1.75.
__device__ __forceinline__ int mx_scale_exp(float a) {
    const uint32_t b = __float_as_uint(fmaxf(a, 1e-4f));
    const int e = (int)(b >> 23) - 127;
    return e - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
}

// A wave normalises a row at a time, rows taken grid-stride by up to
// kNormWaves waves (more than are resident, for balance). Lane l owns 8-channel
// chunks l, l + 64, ...; the row's sum of squares is a wave reduction and a
// 32-channel group is 4 consecutive lanes. When the row fits (kChunks > 0 chunks
// per lane) it stays in registers between the two passes, every load of a row is
// issued before the first wait, and the gain is staged once per workgroup in
// LDS; the register budget leaves room for four waves per SIMD, which keeps a
// whole 4096-row batch in flight. Every access is a raw buffer access whose
// range is the row (or zero for an absent output), so masked lanes and absent
// outputs cost no branch: the body is straight-line and the compiler's
// memory-counter waits stay exact. Wider rows (kChunks == 0) stream the row
// twice and read the gain from memory.
constexpr int kNormRows = kNormBlock / 64;   // waves per workgroup
constexpr int kNormWaves = 8192;             // at most 32 waves per CU on 256 CUs
// float4 of the staged gain each thread loads: 2 per 8-channel chunk
__host__ __device__ constexpr int norm_gain_per_thread(int chunks) { return (chunks * 128 + kNormBlock - 1) / kNormBlock; }
template <bool kBf16>
constexpr int kNormMaxChunks = kBf16 ? 16 : 8;   // at most 64 VGPRs of row per lane
// s_waitcnt immediate that waits for vmcnt <= n only (vmcnt in bits 3:0 and
// 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
__host__ __device__ constexpr int waitcnt_vm(int n) { return ((n >> 4) << 14) | (0xF << 8) | (7 << 4) | (n & 15); }

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// 8 channels as loaded: bf16 one 16-byte word, fp32 two.
template <bool kBf16>
struct NormChunk {
    uint4 w[kBf16 ? 1 : 2];

    __device__ __forceinline__ static uint32_t word(const uint4& u, int i) {
        return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
    }
    __device__ __forceinline__ float get(int i) const {   // i is a compile-time constant after unrolling
        if constexpr (kBf16) {
            const uint32_t u = word(w[0], i >> 1);
            return (i & 1) ? bf16_hi(u) : bf16_lo(u);
        } else {
            return __uint_as_float(word(w[i >> 2], i & 3));
        }
    }
};

// Buffer resources of one row: x (read), y_norm, q and scale (written). A row
// past n, or an output not asked for, gets an empty range.
struct NormRowRsrc {
    __amdgpu_buffer_rsrc_t x, y, q, s;
};

template <bool kBf16>
__device__ __forceinline__ NormRowRsrc norm_row_rsrc(const void* x, void* y_norm, uint8_t* q, uint8_t* scale,
                                                     int64_t t, int64_t n, int64_t d) {
    constexpr int64_t kElem = kBf16 ? 2 : 4;
    const bool ok = t < n;
    const int64_t tt = ok ? t : 0;
    NormRowRsrc r;
    r.x = make_rsrc(static_cast<const uint8_t*>(x) + tt * d * kElem, ok ? d * kElem : 0);
    r.y = make_rsrc(y_norm ? static_cast<uint8_t*>(y_norm) + tt * d * kElem : nullptr, ok && y_norm ? d * kElem : 0);
    r.q = make_rsrc(q ? q + tt * d : nullptr, ok && q ? d : 0);
    r.s = make_rsrc(q ? scale + tt * (d / 32) : nullptr, ok && q ? d / 32 : 0);
    return r;
}

// Byte offset of chunk c within a row, or kOffMasked past the row end.
template <bool kBf16>
__device__ __forceinline__ uint32_t norm_chunk_off(uint32_t c, uint32_t nch) {
    return c < nch ? c * (kBf16 ? 16u : 32u) : kOffMasked;
}

template <bool kBf16>
__device__ __forceinline__ void norm_load(NormChunk<kBf16>& xc, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    xc.w[0] = buf_load16(r, off, 0);
    if constexpr (!kBf16) xc.w[1] = buf_load16(r, off + 16, 0);   // a masked offset stays out of range
}

template <bool kBf16, int kChunks>
__device__ __forceinline__ void norm_load_row(NormChunk<kBf16> (&xc)[kChunks], __amdgpu_buffer_rsrc_t r,
                                              uint32_t lane, uint32_t nch) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) norm_load<kBf16>(xc[i], r, norm_chunk_off<kBf16>(lane + i * 64, nch));
}

// Sum of squares of a chunk (chunks past the row end were loaded as zeros).
// bf16: one dot2 per packed word (the squares of bf16 values are exact in fp32).
template <bool kBf16>
__device__ __forceinline__ void norm_sumsq(const NormChunk<kBf16>& xc, float& ss) {
    if constexpr (kBf16) {
        const uint32_t w[4] = {xc.w[0].x, xc.w[0].y, xc.w[0].z, xc.w[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x2_t b = __builtin_bit_cast(bf16x2_t, w[i]);
            ss = __builtin_amdgcn_fdot2_f32_bf16(b, b, ss, false);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(xc.get(e), xc.get(e), ss);
    }
}

__device__ __forceinline__ void buf_store8(u32x2_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)voff, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 1");   // the same two wait states as buf_store16
    __builtin_amdgcn_sched_barrier(0);
}

// Pass 2 for chunk c of a row: scale by r and the gain (g0, g1), round to the
// row dtype, store the normalised values, and cast the chunk's share of its
// 32-channel group. Stores of a chunk past the row end use a masked offset; a
// dead lane's quad is all dead (d % 32 == 0 when casting), so whatever it
// computes is dropped.
template <bool kBf16>
__device__ __forceinline__ void norm_cast_chunk(const NormChunk<kBf16>& xc, float4 g0, float4 g1, float r,
                                                uint32_t c, uint32_t nch, const NormRowRsrc& rr) {
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    Vec8<kBf16> v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v.v[i] = xc.get(i) * r * gv[i];
    // amax of the rounded values: rounding to nearest is monotonic, so it is the
    // rounded amax of the fp32 values
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v.v[i]));
    if constexpr (kBf16) a = bf16_lo(pack_bf16x2(a, 0.f));
    v.round();   // the normalised row in its dtype
    const uint32_t off = norm_chunk_off<kBf16>(c, nch);
    if constexpr (kBf16) {
        buf_store16(v.raw, rr.y, off, 0);
    } else {
        buf_store16(make_uint4(__float_as_uint(v.v[0]), __float_as_uint(v.v[1]), __float_as_uint(v.v[2]),
                               __float_as_uint(v.v[3])),
                    rr.y, off, 0);
        buf_store16(make_uint4(__float_as_uint(v.v[4]), __float_as_uint(v.v[5]), __float_as_uint(v.v[6]),
                               __float_as_uint(v.v[7])),
                    rr.y, off + 16, 0);
    }
    a = fmaxf(a, dpp<kQuadSwap1>(a));
    a = fmaxf(a, dpp<kQuadSwap2>(a));
    const int k = mx_scale_exp(a);
    // |v| <= amax <= 448 * 2^k, so the scaled values need no clamp. The hardware
    // packs (two codes per instruction) round v / 2^k to the nearest OCP E4M3
    // code, ties to the even code, sign kept, the subnormal codes (multiples of
    // 2^-9 below 2^-6) included; the bf16 form reads the packed words directly.
    uint32_t w0, w1;
    if constexpr (kBf16) {
        const float sc = __uint_as_float((uint32_t)(127 + k) << 23);   // 2^k, exact
        typedef short s16x2_t __attribute__((ext_vector_type(2)));
        const uint32_t raw[4] = {v.raw.x, v.raw.y, v.raw.z, v.raw.w};
        s16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s16x2_t{0, 0}, __builtin_bit_cast(bf16x2_t, raw[0]),
                                                               sc, false);
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(bf16x2_t, raw[1]), sc, true);
        s16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s16x2_t{0, 0}, __builtin_bit_cast(bf16x2_t, raw[2]),
                                                               sc, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(bf16x2_t, raw[3]), sc, true);
        w0 = __builtin_bit_cast(uint32_t, lo);
        w1 = __builtin_bit_cast(uint32_t, hi);
    } else {
        const float inv_s = __uint_as_float((uint32_t)(127 - k) << 23);   // 2^-k, exact
        w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v.v[0] * inv_s, v.v[1] * inv_s, 0, false);
        w0 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v.v[2] * inv_s, v.v[3] * inv_s, (int)w0, true);
        w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v.v[4] * inv_s, v.v[5] * inv_s, 0, false);
        w1 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v.v[6] * inv_s, v.v[7] * inv_s, (int)w1, true);
    }
    buf_store8(u32x2_t{w0, w1}, rr.q, c < nch ? c * 8 : kOffMasked);
    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)(k + 127), rr.s, (c < nch && (c & 3) == 0) ? c / 4 : kOffMasked,
                                         0, 0);
}

template <bool kBf16, int kChunks>
__device__ __forceinline__ void norm_process_row(const NormChunk<kBf16> (&xc)[kChunks], const float4* gain_lds,
                                                 float eps, int64_t d, uint32_t lane, uint32_t nch,
                                                 const NormRowRsrc& rr) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) norm_sumsq<kBf16>(xc[i], ss);
    const float r = 1.0f / sqrtf(wave_sum(ss) / (float)d + eps);
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const uint32_t c = lane + i * 64;
        const uint32_t cg = c < nch ? c : nch - 1;
        norm_cast_chunk<kBf16>(xc[i], gain_lds[2 * cg], gain_lds[2 * cg + 1], r, c, nch, rr);
    }
}

template <bool kBf16, int kChunks>
__global__ __launch_bounds__(kNormBlock) void rmsnorm_mxfp8_kernel(const void* __restrict__ x,
                                                                  const float* __restrict__ gain, int64_t n,
                                                                  int64_t d, float eps, void* __restrict__ y_norm,
                                                                  uint8_t* __restrict__ q,
                                                                  uint8_t* __restrict__ scale) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * kNormRows;
    const uint32_t nch = (uint32_t)(d / 8);
    int64_t ta = (int64_t)blockIdx.x * kNormRows + wave;
    if constexpr (kChunks > 0) {
        extern __shared__ float4 gain_lds[];   // kGainPer * kNormBlock entries: the gain, padded
        constexpr int kGainPer = norm_gain_per_thread(kChunks);
        // Stage the gain straight into LDS (a 16-byte load per lane, written at
        // the wave's base + 16 * lane), ahead of the row loads; entries past the
        // gain repeat its last float4 and are never read.
        const uint32_t ng = nch * 2;
#pragma unroll
        for (int j = 0; j < kGainPer; ++j) {
            const uint32_t k = threadIdx.x + j * kNormBlock;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(reinterpret_cast<const float4*>(gain) +
                                                                (k < ng ? k : ng - 1)),
                (__attribute__((address_space(3))) void*)(gain_lds + j * kNormBlock + wave * 64), 16, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the staging loads ahead of the row loads
        constexpr int kLoadsPerRow = kChunks * (kBf16 ? 1 : 2);
        NormChunk<kBf16> xc[kChunks];
        NormRowRsrc rr = norm_row_rsrc<kBf16>(x, y_norm, q, scale, ta, n, d);
        norm_load_row<kBf16, kChunks>(xc, rr.x, lane, nch);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoadsPerRow));   // the staging loads (issued first) are done
        __syncthreads();                                        // ... in every wave
        while (ta < n) {
            norm_process_row<kBf16, kChunks>(xc, gain_lds, eps, d, lane, nch, rr);
            ta += nw;
            if (ta >= n) break;
            rr = norm_row_rsrc<kBf16>(x, y_norm, q, scale, ta, n, d);
            norm_load_row<kBf16, kChunks>(xc, rr.x, lane, nch);
        }
    } else {
        const float4* gv = reinterpret_cast<const float4*>(gain);
        for (; ta < n; ta += nw) {
            const NormRowRsrc rr = norm_row_rsrc<kBf16>(x, y_norm, q, scale, ta, n, d);
            NormChunk<kBf16> xc;
            float ss = 0.f;
            for (uint32_t c = lane; c < nch; c += 64) {
                norm_load<kBf16>(xc, rr.x, norm_chunk_off<kBf16>(c, nch));
                norm_sumsq<kBf16>(xc, ss);
            }
            const float r = 1.0f / sqrtf(wave_sum(ss) / (float)d + eps);
            for (uint32_t c0 = 0; c0 < nch; c0 += 64) {   // uniform trip count: quads stay whole
                const uint32_t c = c0 + lane;
                const uint32_t cg = c < nch ? c : nch - 1;
                norm_load<kBf16>(xc, rr.x, norm_chunk_off<kBf16>(c, nch));
                norm_cast_chunk<kBf16>(xc, gv[2 * cg], gv[2 * cg + 1], r, c, nch, rr);
            }
        }
    }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// ------------------------------------------------------------------- launchers
constexpr int kF32Unit = 128;   // pass_kernel slices are whole 128-channel units

PassPlan plan_pass(int64_t n, int64_t d, bool bf16) {
    PassPlan p{};
    // bf16 sweep: 64-token groups (128 from kWideSweepTokens tokens on), slices of
    // whole 64-channel steps, ~256 workgroups (one per CU); fp32 pass_kernel:
    // 64-token tiles, 128-channel units
    p.wide = bf16 && n >= kWideSweepTokens;
    const int tok = bf16 ? (p.wide ? kS2Tok : kSwTok) : kTokWG;
    const int unit = bf16 ? kStep : kF32Unit;
    p.tiles = ceil_div(n, tok);
    p.nchunks = (int)ceil_div(d, kChunk);
    const int nunits = (int)ceil_div(d, unit);
    const int64_t target_groups = bf16 ? kSweepTargetGroups : kPassTargetGroups;
    int64_t ns = ceil_div(target_groups, p.tiles > 0 ? p.tiles : 1);
    if (ns < 1) ns = 1;
    if (ns > nunits) ns = nunits;
    if (ns > 8 * kFinWaveRounds) ns = 8 * kFinWaveRounds;   // what the wave finalize reduces
    p.chunks_per_split = (int)ceil_div(nunits, ns) * (unit / kChunk);
    p.nsplit = (int)ceil_div(p.nchunks, p.chunks_per_split);
    // partial rows: nsplit x n x 32 floats
    p.workspace_bytes = (size_t)p.nsplit * (size_t)n * kPart * sizeof(float);
    return p;
}

// Work-items of the largest grid the four-stream launchers form for (n, d), over
// every entry point and both stream dtypes: the split (a lane per token), the
// collapse and expand (a lane per 8 channels), the sweeps, and the finalize (16
// lanes per token, or a wave per token when there are more than 8 slices).
int64_t max_launch_items(int64_t n, int64_t d) {
    int64_t m = ceil_div(n, kSplitBlock) * kSplitBlock;
    const int64_t ew = ceil_div(n * (d / 8), kEwBlock) * kEwBlock;
    if (ew > m) m = ew;
    for (int k = 0; k < 2; ++k) {
        const PassPlan p = plan_pass(n, d, k == 1);
        const int64_t sweep = p.tiles * p.nsplit * (k == 1 ? kSwBlock : kPassBlock);
        const int64_t fin = p.nsplit > kFin16Slices ? ceil_div(n, kFinBlock / 64) * kFinBlock
                                                    : ceil_div(n * 16, kFinBlock) * kFinBlock;
        if (sweep > m) m = sweep;
        if (fin > m) m = fin;
    }
    return m;
}

size_t workspace_bytes(int64_t n, int64_t d) {
    const PassPlan a = plan_pass(n, d, false), b = plan_pass(n, d, true);
    return a.workspace_bytes > b.workspace_bytes ? a.workspace_bytes : b.workspace_bytes;
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
    const bool stream_out = n * kHC * d * (bf16 ? 2 : 4) >= kStreamOutBytes;
    if (bf16 && stream_out)
        hipLaunchKernelGGL((post_kernel<true, true>), grid, dim3(kEwBlock), 0, stream, f, res, post, comb, n, d, out);
    else if (bf16)
        hipLaunchKernelGGL((post_kernel<true, false>), grid, dim3(kEwBlock), 0, stream, f, res, post, comb, n, d, out);
    else if (stream_out)
        hipLaunchKernelGGL((post_kernel<false, true>), grid, dim3(kEwBlock), 0, stream, f, res, post, comb, n, d, out);
    else
        hipLaunchKernelGGL((post_kernel<false, false>), grid, dim3(kEwBlock), 0, stream, f, res, post, comb, n, d,
                           out);
    return hipGetLastError();
}

namespace {
template <bool kPost, bool kPre>
void launch_sweep_t(const PassArgs& a, const PassPlan& p, hipStream_t stream) {
    if (p.wide)
        hipLaunchKernelGGL((bf16_sweep2_kernel<kPost, kPre>), dim3((unsigned)(p.tiles * p.nsplit)), dim3(kSwBlock),
                           0, stream, a);
    else if (p.chunks_per_split <= kStepKb)   // every slice one step
        hipLaunchKernelGGL((bf16_sweep_kernel<kPost, kPre, true>), dim3((unsigned)(p.tiles * p.nsplit)),
                           dim3(kSwBlock), 0, stream, a);
    else
        hipLaunchKernelGGL((bf16_sweep_kernel<kPost, kPre, false>), dim3((unsigned)(p.tiles * p.nsplit)),
                           dim3(kSwBlock), 0, stream, a);
}

template <bool kPost, bool kPre>
void launch_pass_t(const PassArgs& a, const PassPlan& p, hipStream_t stream) {
    hipLaunchKernelGGL((pass_kernel<kPost, kPre>), dim3((unsigned)(p.tiles * p.nsplit)), dim3(kPassBlock), 0,
                       stream, a);
}
}  // namespace

template <bool kBf16, int kChunks>
void launch_norm(dim3 grid, const void* x, const float* gain, int64_t n, int64_t d, float eps, void* y_norm,
                 uint8_t* q, uint8_t* scale, hipStream_t stream) {
    const size_t lds = (size_t)norm_gain_per_thread(kChunks) * kNormBlock * sizeof(float4);   // the staged gain
    hipLaunchKernelGGL((rmsnorm_mxfp8_kernel<kBf16, kChunks>), grid, dim3(kNormBlock), lds, stream, x, gain, n, d,
                       eps, y_norm, q, scale);
}

template <bool kBf16>
void launch_norm_dtype(dim3 grid, const void* x, const float* gain, int64_t n, int64_t d, float eps, void* y_norm,
                       uint8_t* q, uint8_t* scale, hipStream_t stream) {
    // chunks per lane, rounded up to an even count (one instance per even count)
    const int64_t need = ceil_div(d / 8, 64);
    switch (need <= kNormMaxChunks<kBf16> ? (need + 1) / 2 * 2 : 0) {
        case 2: return launch_norm<kBf16, 2>(grid, x, gain, n, d, eps, y_norm, q, scale, stream);
        case 4: return launch_norm<kBf16, 4>(grid, x, gain, n, d, eps, y_norm, q, scale, stream);
        case 6: return launch_norm<kBf16, 6>(grid, x, gain, n, d, eps, y_norm, q, scale, stream);
        case 8: return launch_norm<kBf16, 8>(grid, x, gain, n, d, eps, y_norm, q, scale, stream);
        case 10: return launch_norm<kBf16, kBf16 ? 10 : 0>(grid, x, gain, n, d, eps, y_norm, q, scale, stream);
        case 12: return launch_norm<kBf16, kBf16 ? 12 : 0>(grid, x, gain, n, d, eps, y_norm, q, scale, stream);
        case 14: return launch_norm<kBf16, kBf16 ? 14 : 0>(grid, x, gain, n, d, eps, y_norm, q, scale, stream);
        case 16: return launch_norm<kBf16, kBf16 ? 16 : 0>(grid, x, gain, n, d, eps, y_norm, q, scale, stream);
        default: return launch_norm<kBf16, 0>(grid, x, gain, n, d, eps, y_norm, q, scale, stream);
    }
}

hipError_t launch_rmsnorm_mxfp8(const void* x, bool bf16, const float* gain, int64_t n, int64_t d, float eps,
                                void* y_norm, uint8_t* q, uint8_t* scale, hipStream_t stream) {
    const dim3 grid((unsigned)ceil_div(n < kNormWaves ? n : kNormWaves, kNormRows));   // rows grid-stride
    if (bf16)
        launch_norm_dtype<true>(grid, x, gain, n, d, eps, y_norm, q, scale, stream);
    else
        launch_norm_dtype<false>(grid, x, gain, n, d, eps, y_norm, q, scale, stream);
    return hipGetLastError();
}

hipError_t launch_pass_and_finalize(const PassRequest& r, hipStream_t stream) {
    const PassPlan p = plan_pass(r.n, r.d, r.bf16);
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
        if (post && pre) launch_sweep_t<true, true>(a, p, stream);
        else if (post) launch_sweep_t<true, false>(a, p, stream);
        else if (pre) launch_sweep_t<false, true>(a, p, stream);
        else launch_sweep_t<false, false>(a, p, stream);
    } else {
        if (post && pre) launch_pass_t<true, true>(a, p, stream);
        else if (post) launch_pass_t<true, false>(a, p, stream);
        else if (pre) launch_pass_t<false, true>(a, p, stream);
        else launch_pass_t<false, false>(a, p, stream);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (p.nsplit > kFin16Slices)   // many slices: a wave per token keeps every partial load in flight
        hipLaunchKernelGGL(finalize_wave_kernel, dim3((unsigned)ceil_div(r.n, kFinBlock / 64)), dim3(kFinBlock), 0,
                           stream, f);
    else
        hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)ceil_div(r.n * 16, kFinBlock)), dim3(kFinBlock), 0,
                           stream, f);
    return hipGetLastError();
}

}  // namespace hc
