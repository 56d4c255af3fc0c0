// hc_generic.hip -- gfx950 kernels for stream counts other than four (1 <= hc <= 8).
//
// Sources (page titles and sections):
//   atlas "Stream combination", code section: the split kernel is written for any
//       stream count hc and number of rounds; the mix numbers of a token are
//       [pre (hc) | post (hc) | comb (hc x hc, row-major)].
//   atlas "Block", code section: hc_mixes (one RMS statistic over the hc*d
//       flattened streams, projection scaled after the dot products), hc_pre,
//       hc_post for hc_mult streams.
//
// Four streams take the single-pass kernels of hc_kernels.hip. Here every step is
// a kernel of its own; the fused boundary is their composition:
//   split_generic_kernel    a wave per token; lane j*hc + k owns comb[j][k], rows
//                           and columns are summed with cross-lane reads
//                           (split_butterfly_kernel: butterflies for two and
//                           eight streams).
//   pre_generic_kernel      collapse, one lane per (token, 8 channels), a wave
//                           per token and 512 channels.
//   post_generic_kernel     expand + combine, the same mapping; in a fused step
//                           with an expand it also collapses the new streams.
//   mixes_partial_kernel    64 tokens x one slice of the flattened hc*d axis per
//                           workgroup: the (2+hc)*hc partial dot products (fp32
//                           MFMA) and the partial sum of squares, from LDS tiles
//                           of 64 columns (fp32 streams).
//   mixes_partial_bf16_kernel  the same partial rows for bf16 streams: 128 tokens
//                           per workgroup, bf16 MFMAs on the exact stream values
//                           and on the weights split into three bf16 terms
//                           (one to three streams).
//   mixes_wide_bf16_kernel  the same for five to eight bf16 streams: 256 tokens
//                           per workgroup, staging and multiplying waves meeting
//                           at one barrier per tile.
//   mixes_finalize_kernel   a wave per token: partial rows summed over the slices
//                           in order, scaled by the RMS statistic.
//
// Arithmetic is fp32 throughout; bf16 outputs are rounded to nearest-even.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "hc_internal.h"

namespace hc {
namespace {

typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kGBlock = 256;
constexpr int kGTok = 64;       // tokens per projection workgroup (16 per wave)
constexpr int kGCols = 64;      // flattened columns per LDS tile
// Slices of the flattened axis, at most. Few tokens take many slices: that fills
// the GPU and keeps each slice's fp32 accumulation chain short (at d = 2^20 and
// eight streams, 256 slices leave 32768 flattened columns per chain).
constexpr int kGMaxSplit = 256;

__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + __expf(-z)); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){a, b}, bf16x2_t));
}

// Eight consecutive elements at element index idx (a multiple of 8), as fp32.
template <bool kBf16>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float (&v)[8]) {
    if constexpr (kBf16) {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(u[i] << 16);
            v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
        const float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

// Stores eight fp32 values rounded once to the element type; kStream: with
// non-temporal stores (to HBM, not kept in the caches).
typedef unsigned int u32x4_s __attribute__((ext_vector_type(4)));
template <bool kBf16, bool kStream = false>
__device__ __forceinline__ void store8(void* base, int64_t idx, const float (&v)[8]) {
    if constexpr (kBf16) {
        const u32x4_s w = {pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
        u32x4_s* p = reinterpret_cast<u32x4_s*>(static_cast<uint16_t*>(base) + idx);
        if constexpr (kStream) __builtin_nontemporal_store(w, p);
        else *p = w;
    } else {
        const u32x4_s a = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
        const u32x4_s b = {__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])};
        u32x4_s* p = reinterpret_cast<u32x4_s*>(static_cast<float*>(base) + idx);
        if constexpr (kStream) {
            __builtin_nontemporal_store(a, p);
            __builtin_nontemporal_store(b, p + 1);
        } else {
            p[0] = a;
            p[1] = b;
        }
    }
}

// ---------------------------------------------------------------- split
// Row j of the comb lives in lanes j*hc .. j*hc + hc-1. Sums run over k (rows)
// or j (columns) in ascending order. Lanes past hc*hc compute on row 0 and store
// nothing.
__device__ __forceinline__ float row_sum_g(float c, int j, int hc) {
    float s = 0.f;
    for (int k = 0; k < hc; ++k) s += __shfl(c, j * hc + k);
    return s;
}
__device__ __forceinline__ float col_sum_g(float c, int k, int hc) {
    float s = 0.f;
    for (int j = 0; j < hc; ++j) s += __shfl(c, j * hc + k);
    return s;
}

// The split of one token by one wave. mix(i) returns the token's mix i; every
// lane of the wave calls it (it may read other lanes' registers).
template <class Mix>
__device__ __forceinline__ void split_generic_wave(const Mix& mix, const float* __restrict__ scale,
                                                   const float* __restrict__ base, int64_t t, int hc, int iters,
                                                   float eps, float* __restrict__ pre, float* __restrict__ post,
                                                   float* __restrict__ comb) {
    const int lane = threadIdx.x & 63;
    const int hc2 = hc * hc;
    const bool cl = lane < hc2;
    const int j = cl ? lane / hc : 0;
    const int k = cl ? lane - j * hc : 0;
    const int ci = 2 * hc + (cl ? lane : 0);
    const float mp = mix(lane < 2 * hc ? lane : 0);   // pre / post logit of lanes 0 .. 2 hc - 1
    float c = mix(ci) * scale[2] + base[ci];
    // row softmax (max subtracted), + eps; then the column step
    float mx = -INFINITY;
    for (int kk = 0; kk < hc; ++kk) mx = fmaxf(mx, __shfl(c, j * hc + kk));
    c = __expf(c - mx);
    c = c * __builtin_amdgcn_rcpf(row_sum_g(c, j, hc)) + eps;
    c *= __builtin_amdgcn_rcpf(col_sum_g(c, k, hc) + eps);
    for (int it = 1; it < iters; ++it) {
        c *= __builtin_amdgcn_rcpf(row_sum_g(c, j, hc) + eps);
        c *= __builtin_amdgcn_rcpf(col_sum_g(c, k, hc) + eps);
    }
    if (cl) comb[t * hc2 + lane] = c;
    if (lane < hc)
        pre[t * hc + lane] = sigmoid_f(mp * scale[0] + base[lane]) + eps;
    else if (lane < 2 * hc)
        post[t * hc + lane - hc] = 2.0f * sigmoid_f(mp * scale[1] + base[lane]);
}

__global__ __launch_bounds__(kGBlock) void split_generic_kernel(const float* __restrict__ mixes,
                                                                const float* __restrict__ scale,
                                                                const float* __restrict__ base, int64_t n,
                                                                int hc, int iters, float eps,
                                                                float* __restrict__ pre, float* __restrict__ post,
                                                                float* __restrict__ comb) {
    const int64_t t = (int64_t)blockIdx.x * (kGBlock / 64) + (threadIdx.x >> 6);
    if (t >= n) return;   // a whole wave leaves together
    const float* m = mixes + t * (2 + hc) * hc;
    split_generic_wave([&](int i) { return m[i]; }, scale, base, t, hc, iters, eps, pre, post, comb);
}

// Two or eight streams: a comb row is kH aligned lanes and a column is lanes
// k, k + kH, ..., so the sums are butterflies instead of kH cross-lane reads
// each. Two streams: a row is a lane pair (quad swap by 1) and a column lanes k
// and k + 2 (quad swap by 2). Eight streams: a row takes two quad swaps and a
// half-row mirror (DPP); a column a rotation by 8 within each 16-lane row (DPP),
// then sums across 16-lane rows and 32-lane halves with gfx950's lane swaps
// (v_permlane16_swap / v_permlane32_swap: with both operands the same value, the
// two results hold each lane's own value and its partner's, in an order that
// depends on the row, so their sum is the lane's value plus its partner's).
// Every partner pair adds the same two numbers, so all lanes of a row (column)
// end with the same sum. Lanes past kH * kH
// compute on row 0 and store nothing. Otherwise the same steps as
// split_generic_kernel.
template <int kCtrl>
__device__ __forceinline__ float dpp_g(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}
constexpr int kDppQuad1 = 0xb1, kDppQuad2 = 0x4e, kDppHalfMirror = 0x141, kDppRor8 = 0x128;

template <int kH>
__device__ __forceinline__ float row_sum_b(float v) {
    v += dpp_g<kDppQuad1>(v);
    if constexpr (kH == 8) {
        v += dpp_g<kDppQuad2>(v);
        v += dpp_g<kDppHalfMirror>(v);
    }
    return v;
}
template <int kH>
__device__ __forceinline__ float row_max_b(float v) {
    v = fmaxf(v, dpp_g<kDppQuad1>(v));
    if constexpr (kH == 8) {
        v = fmaxf(v, dpp_g<kDppQuad2>(v));
        v = fmaxf(v, dpp_g<kDppHalfMirror>(v));
    }
    return v;
}
// v plus the value of lane l ^ 16 (kSpan 16) or l ^ 32 (kSpan 32), every lane active
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
template <int kH>
__device__ __forceinline__ float col_sum_b(float v) {
    if constexpr (kH == 2) return v + dpp_g<kDppQuad2>(v);
    v += dpp_g<kDppRor8>(v);
    v = add_partner<16>(v);
    return add_partner<32>(v);
}

template <int kH, class Mix>
__device__ __forceinline__ void split_butterfly_wave(const Mix& mix, const float* __restrict__ scale,
                                                     const float* __restrict__ base, int64_t t, int iters, float eps,
                                                     float* __restrict__ pre, float* __restrict__ post,
                                                     float* __restrict__ comb) {
    // No contraction: the compiler would fuse a lane's own product into the first
    // add of a column sum, while its partner's term arrives rounded, so the lanes
    // of a column would not add the same two numbers; the fused multiply-adds
    // meant here are written out.
#pragma clang fp contract(off)
    static_assert(kH == 2 || kH == 8, "butterflies for two or eight streams");
    const int lane = threadIdx.x & 63;
    const bool cl = lane < kH * kH;
    const int ci = 2 * kH + (cl ? lane : lane % kH);
    const float mp = mix(lane < 2 * kH ? lane : 0);   // pre / post logit of lanes 0 .. 2 kH - 1
    float c = fmaf(mix(ci), scale[2], base[ci]);
    c = __expf(c - row_max_b<kH>(c));
    c = fmaf(c, __builtin_amdgcn_rcpf(row_sum_b<kH>(c)), eps);
    c *= __builtin_amdgcn_rcpf(col_sum_b<kH>(c) + eps);
    for (int it = 1; it < iters; ++it) {
        c *= __builtin_amdgcn_rcpf(row_sum_b<kH>(c) + eps);
        c *= __builtin_amdgcn_rcpf(col_sum_b<kH>(c) + eps);
    }
    if (cl) comb[t * kH * kH + lane] = c;
    if (lane < kH)
        pre[t * kH + lane] = sigmoid_f(fmaf(mp, scale[0], base[lane])) + eps;
    else if (lane < 2 * kH)
        post[t * kH + lane - kH] = 2.0f * sigmoid_f(fmaf(mp, scale[1], base[lane]));
}

template <int kH>
__global__ __launch_bounds__(kGBlock) void split_butterfly_kernel(const float* __restrict__ mixes,
                                                                  const float* __restrict__ scale,
                                                                  const float* __restrict__ base, int64_t n,
                                                                  int iters, float eps, float* __restrict__ pre,
                                                                  float* __restrict__ post,
                                                                  float* __restrict__ comb) {
    const int64_t t = (int64_t)blockIdx.x * (kGBlock / 64) + (threadIdx.x >> 6);
    if (t >= n) return;   // a whole wave leaves together
    const float* m = mixes + t * (2 + kH) * kH;
    split_butterfly_wave<kH>([&](int i) { return m[i]; }, scale, base, t, iters, eps, pre, post, comb);
}

// --------------------------------------------------------- collapse / expand
// A wave covers one token and 64 of its 8-channel chunks (wave (t, wc) of the
// grid owns chunks wc*64 + lane), so the token's coefficients are wave-uniform
// and read once per wave through the scalar cache.
__device__ __forceinline__ bool wave_token(int64_t n, int64_t per_tok, int64_t& t, int64_t& e) {
    const int64_t wpt = (per_tok + 63) >> 6;   // waves per token
    const int64_t gw = (int64_t)blockIdx.x * (kGBlock / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    t = gw / wpt;
    const int64_t c = (gw - t * wpt) * 64 + (threadIdx.x & 63);
    e = c << 3;
    return t < n && c < per_tok;
}

int64_t wave_grid(int64_t n, int64_t d) { return (n * (((d >> 3) + 63) >> 6) + kGBlock / 64 - 1) / (kGBlock / 64); }

template <bool kBf16>
__global__ __launch_bounds__(kGBlock) void pre_generic_kernel(const void* __restrict__ x,
                                                              const float* __restrict__ pre_mix, int64_t n,
                                                              int hc, int64_t d, void* __restrict__ y) {
    int64_t t, e;
    if (!wave_token(n, d >> 3, t, e)) return;
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;
    for (int j = 0; j < hc; ++j) {
        const float w = pre_mix[t * hc + j];
        float v[8];
        load8<kBf16>(x, (t * hc + j) * d + e, v);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(w, v[c], acc[c]);
    }
    store8<kBf16>(y, t * d + e, acc);
}

// The values a store8 of v writes, read back as fp32.
template <bool kBf16>
__device__ __forceinline__ void stored8(const float (&v)[8], float (&r)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (kBf16) {
            const uint32_t w = pack2(v[2 * i], v[2 * i + 1]);
            r[2 * i] = __uint_as_float(w << 16);
            r[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
        } else {
            r[2 * i] = v[2 * i];
            r[2 * i + 1] = v[2 * i + 1];
        }
    }
}

// Every stream of the lane's 8 channels is read before any is written, so the
// output may be the residual itself. kCollapse: the new streams, as stored, are
// also collapsed with pre_mix into y (ascending stream, one fma each, as the
// collapse of the projection kernels and pre_generic_kernel do).
template <bool kBf16, bool kStream, bool kCollapse>
__global__ __launch_bounds__(kGBlock) void post_generic_kernel(const void* __restrict__ f, const void* res,
                                                               const float* __restrict__ post,
                                                               const float* __restrict__ comb, int64_t n, int hc,
                                                               int64_t d, void* out, const float* __restrict__ pre_mix,
                                                               void* __restrict__ y) {
    int64_t t, e;
    if (!wave_token(n, d >> 3, t, e)) return;
    float fv[8], rv[kMaxHC][8], yacc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) yacc[c] = 0.f;
    load8<kBf16>(f, t * d + e, fv);
#pragma unroll
    for (int j = 0; j < kMaxHC; ++j)
        if (j < hc) load8<kBf16>(res, (t * hc + j) * d + e, rv[j]);
#pragma unroll
    for (int k = 0; k < kMaxHC; ++k) {
        if (k >= hc) break;
        const float pk = post[t * hc + k];
        float o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = pk * fv[c];
#pragma unroll
        for (int j = 0; j < kMaxHC; ++j) {
            if (j >= hc) break;
            const float cjk = comb[(t * hc + j) * hc + k];
#pragma unroll
            for (int c = 0; c < 8; ++c) o[c] = fmaf(cjk, rv[j][c], o[c]);
        }
        store8<kBf16, kStream>(out, (t * hc + k) * d + e, o);
        if constexpr (kCollapse) {
            const float pk = pre_mix[t * hc + k];
            float r[8];
            stored8<kBf16>(o, r);
#pragma unroll
            for (int c = 0; c < 8; ++c) yacc[c] = fmaf(pk, r[c], yacc[c]);
        }
    }
    if constexpr (kCollapse) store8<kBf16>(y, t * d + e, yacc);
}

// ------------------------------------------------------------- projection
// fp32 streams. Workgroup (tile, slice): tokens tile*64 .. +64 and flattened
// columns [slice * cols_per_split, +cols_per_split), walked in tiles of 64
// columns staged in LDS (the streams and the hc_fn rows; rows of the hc_fn tile
// past the last mix are zero). The next tile is fetched into registers
// while the current one is multiplied. Wave w multiplies its 16 tokens by the R
// 16-wide column tiles of hc_fn with v_mfma_f32_16x16x4f32 (exact fp32 products,
// fp32 accumulation): lane l (row l % 16, group g = l / 16) feeds, at each of the
// 16 MFMA steps of a 64-column tile, column 16 g + step to both operands, so its
// operands are 128-bit LDS reads of 4 consecutive columns. The sum of squares is
// accumulated by the same lanes on the VALU and summed over the 4 groups at the
// end. Output: one partial row per (slice, token): the (2+hc)hc dots, then the
// sum of squares.
constexpr int kGRow = kGCols + 4;   // LDS row stride (floats)

typedef float floatx4_g __attribute__((ext_vector_type(4)));

// One 64-column tile as fetched from memory, held in registers until it is
// written to LDS: lane tid owns stream columns (tid % 4) * 16 .. +16 of token
// tid / 4, and float4 slots tid + 256 r of the hc_fn tile (16 slots per row, rows
// past the last mix read as zero).
template <int R>
struct GenericStage {
    float4 xv[4];
    float4 wv[R];
};

template <int R>
__device__ __forceinline__ void stage_load(GenericStage<R>& st, const float* x, const float* hc_fn, int64_t n, int M,
                                           int64_t K, int64_t t0, int64_t c0, int64_t c_end) {
    const int tid = threadIdx.x, row = tid >> 2, col = (tid & 3) * 16;
    const int64_t t = t0 + row;
#pragma unroll
    for (int h = 0; h < 2; ++h) {   // two halves of 8 columns; K and the slice bounds are multiples of 8
        const int64_t c = c0 + col + 8 * h;
        const bool ok = t < n && c < c_end;
        const float4* p = reinterpret_cast<const float4*>(x + t * K + c);
        st.xv[2 * h] = ok ? p[0] : make_float4(0.f, 0.f, 0.f, 0.f);
        st.xv[2 * h + 1] = ok ? p[1] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int q = tid + kGBlock * r, i = q / (kGCols / 4), lc = (q % (kGCols / 4)) * 4;
        const int64_t c = c0 + lc;
        st.wv[r] = (i < M && c < c_end) ? *reinterpret_cast<const float4*>(hc_fn + (int64_t)i * K + c)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

template <int R>
__device__ __forceinline__ void stage_store(const GenericStage<R>& st, float* xs, float* ws) {
    const int tid = threadIdx.x, row = tid >> 2, col = (tid & 3) * 16;
    float4* dst = reinterpret_cast<float4*>(xs + row * kGRow + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = st.xv[i];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int q = tid + kGBlock * r, i = q / (kGCols / 4), lc = (q % (kGCols / 4)) * 4;
        *reinterpret_cast<float4*>(ws + i * kGRow + lc) = st.wv[r];
    }
}

template <int R>
__global__ __launch_bounds__(kGBlock) void mixes_partial_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ hc_fn, int64_t n,
                                                                int hc, int64_t d, int cols_per_split,
                                                                int nsplit, float* __restrict__ part, int pg) {
    __shared__ __attribute__((aligned(16))) float xs[kGTok * kGRow];
    __shared__ __attribute__((aligned(16))) float ws[16 * R * kGRow];
    const int M = (2 + hc) * hc;
    const int64_t K = (int64_t)hc * d;
    const int64_t tile = blockIdx.x / nsplit;
    const int slice = (int)(blockIdx.x - tile * nsplit);
    const int64_t t0 = tile * kGTok;
    const int64_t c_begin = (int64_t)slice * cols_per_split;
    const int64_t c_end = c_begin + cols_per_split < K ? c_begin + cols_per_split : K;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    floatx4_g acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = floatx4_g{0.f, 0.f, 0.f, 0.f};
    float ss = 0.f;
    GenericStage<R> st;
    stage_load<R>(st, x, hc_fn, n, M, K, t0, c_begin, c_end);
    for (int64_t c0 = c_begin; c0 < c_end; c0 += kGCols) {
        __syncthreads();   // the previous tile is consumed
        stage_store<R>(st, xs, ws);
        __syncthreads();
        if (c0 + kGCols < c_end)   // the next tile's loads run under this tile's MFMAs
            stage_load<R>(st, x, hc_fn, n, M, K, t0, c0 + kGCols, c_end);
        const float* xa = xs + (w * 16 + r16) * kGRow + 16 * g;
        // the tile's 64 products per dot (and 16 squares per lane) go to fresh
        // accumulators, added to the running ones once per tile: accumulation chains
        // stay one tile long, so the rounding error does not grow with the slice
        floatx4_g tacc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) tacc[r] = floatx4_g{0.f, 0.f, 0.f, 0.f};
        float tss = 0.f;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 a = *reinterpret_cast<const float4*>(xa + 4 * q4);
            float4 b[R];
#pragma unroll
            for (int r = 0; r < R; ++r)
                b[r] = *reinterpret_cast<const float4*>(ws + (r * 16 + r16) * kGRow + 16 * g + 4 * q4);
            const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                tss = fmaf(av[e], av[e], tss);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float bv[4] = {b[r].x, b[r].y, b[r].z, b[r].w};
                    tacc[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], tacc[r], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] += tacc[r];
        ss += tss;
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    // accumulator lane l: tokens 4 g + i (i < 4) of the wave's 16, mix r*16 + r16
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int mix = r * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + w * 16 + 4 * g + i;
            if (t < n && mix < M) part[((int64_t)slice * n + t) * pg + mix] = acc[r][i];
        }
    }
    const int64_t ts = t0 + w * 16 + r16;
    if (g == 0 && ts < n) part[((int64_t)slice * n + ts) * pg + M] = ss;
}

// bf16 streams. The products of bf16 stream values with bf16 numbers are exact
// in fp32, so the projection runs on bf16 MFMAs once each fp32 weight is split
// into three bf16 terms (w ~ hi + mid + lo, about 24 significant bits), each
// multiplied and accumulated in fp32 (hi, then mid, then lo).
//
// Workgroup (tile, slice): 4 waves x kBT 16-token row tiles and a slice of
// 64-channel blocks. Every B operand read from LDS feeds kBT MFMAs and every
// weight fetched from L2 serves 64 kBT tokens: four row tiles when there are
// three or more column tiles of mixes (hc >= 5) and no collapse, else two (few
// weights; or the registers of the collapse).
//
// The slice is walked channel-major in 64-column tiles: block b of stream 0,
// 1, ..., hc-1, then block b + 1. A tile is one contiguous stretch of both the
// streams (x[t][j][64 b ..]) and the flattened hc_fn columns (j d + 64 b ..).
// With the collapse fused (y given), each thread accumulates
// y[t][e] = sum_j pre_mix[t][j] x[t][j][e] over the hc tiles of a block, in
// ascending j with one fma per stream, and stores it rounded once after the
// last; the streams are read once for both.
//
// The hc_fn tile is split once, when it is written to LDS, into three bf16
// planes; the stream tile stays bf16. LDS rows hold 64 columns padded to 144
// bytes, so that 16 consecutive rows read at one column cover distinct banks.
// Per 64-column tile and 32-column k-block, lane l (row r16 = l % 16, k-group
// g = l / 16) reads 8 columns 8 g .. 8 g + 7 of its row tiles' tokens (A) and
// of mix row r*16 + r16 in each plane (B), as the 16x16x32 bf16 MFMA lays out
// its operands. The sum of squares is the diagonal of A times A (exact
// products, fp32 accumulation).
typedef __bf16 bf16x8_g __attribute__((ext_vector_type(8)));
constexpr int kBRow = kGCols + 8;        // LDS row stride of the bf16 tiles (elements)

__host__ __device__ constexpr int bf16_row_tiles(int R, bool pre) { return (R <= 2 || pre) ? 2 : 4; }   // per wave
__host__ __device__ constexpr int bf16_x_slots(int R, bool pre) {
    return 64 * bf16_row_tiles(R, pre) * kGCols / 8 / kGBlock;
}

__device__ __forceinline__ float bf16_lo_g(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_g(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 weights as three packed bf16 pairs: hi = bf16(w), mid = bf16(w - hi),
// lo = bf16(w - hi - mid); both differences are exact in fp32.
__device__ __forceinline__ void split3_pair(float a, float b, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    hi = pack2(a, b);
    const float ra = a - bf16_lo_g(hi), rb = b - bf16_hi_g(hi);
    mid = pack2(ra, rb);
    lo = pack2(ra - bf16_lo_g(mid), rb - bf16_hi_g(mid));
}

// Raw buffer loads: a wave-uniform resource (base, byte range) plus a per-lane
// offset and a wave-uniform scalar offset. The range check covers the per-lane
// offset only, so a lane whose load must return zero gets kOffMaskedG.
typedef unsigned int u32x4_g __attribute__((ext_vector_type(4)));
constexpr uint32_t kOffMaskedG = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_g(const void* base, int64_t bytes) {
    const int64_t b = bytes < 0 ? 0 : (bytes > 0x7ffffff0 ? 0x7ffffff0 : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)b, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4_g v =
        __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, __builtin_amdgcn_readfirstlane((int)soff), 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// One 64-column tile in registers: stream slot p of thread tid is token row
// tid / 8 + 32 p, columns (tid % 8) * 8 .. +8 (8 lanes cover a row's 128 bytes),
// with that token's collapse weight for the tile's stream; hc_fn slot r is row
// tid / 16 + 16 r, columns (tid % 16) * 4 .. +4. Each slot has a resource
// starting at its first row and ending at the last token or mix row, so that
// rows past either read as zero; one lane offset (the row within the slot and
// the column) serves every slot, the tile's column is the scalar offset.
template <int R, bool kPre>
struct Bf16Stage {
    uint4 xw[bf16_x_slots(R, kPre)];
    float pm[kPre ? bf16_x_slots(R, kPre) : 1];
    uint4 wv[R];
};

template <int R, bool kPre>
struct Bf16Src {
    __amdgpu_buffer_rsrc_t x[bf16_x_slots(R, kPre)];
    __amdgpu_buffer_rsrc_t w[R];
    uint32_t xoff, woff;   // lane offsets (bytes)
};

template <int R, bool kPre>
__device__ __forceinline__ void make_src_bf16(Bf16Src<R, kPre>& src, const uint16_t* x, const float* hc_fn,
                                              int64_t n, int M, int64_t K, int64_t t0) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < bf16_x_slots(R, kPre); ++p) {
        const int64_t row0 = t0 + 32 * p;
        src.x[p] = rsrc_g(x + row0 * K, (n - row0) * K * 2);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) src.w[r] = rsrc_g(hc_fn + (int64_t)16 * r * K, (int64_t)(M - 16 * r) * K * 4);
    src.xoff = (uint32_t)((int64_t)(tid >> 3) * K * 2 + (tid & 7) * 16);
    src.woff = (uint32_t)((int64_t)(tid >> 4) * K * 4 + (tid & 15) * 16);
}

// Tile (block b, stream j): flattened columns j d + 64 b .. +64, channels past d read as zero.
template <int R, bool kPre>
__device__ __forceinline__ void stage_load_bf16(Bf16Stage<R, kPre>& st, const Bf16Src<R, kPre>& src,
                                                const float* pre_mix, int64_t n, int hc, int64_t d, int64_t t0,
                                                int64_t b, int j) {
    const int tid = threadIdx.x;
    const int64_t e0 = b * kGCols, c0 = (int64_t)j * d + e0;
    const uint32_t xo = e0 + (tid & 7) * 8 < d ? src.xoff : kOffMaskedG;     // d is a multiple of 8
    const uint32_t wo = e0 + (tid & 15) * 4 < d ? src.woff : kOffMaskedG;
#pragma unroll
    for (int p = 0; p < bf16_x_slots(R, kPre); ++p) st.xw[p] = bload16(src.x[p], xo, (uint32_t)(c0 * 2));
#pragma unroll
    for (int r = 0; r < R; ++r) st.wv[r] = bload16(src.w[r], wo, (uint32_t)(c0 * 4));
    if constexpr (kPre) {
#pragma unroll
        for (int p = 0; p < bf16_x_slots(R, kPre); ++p) {
            const int64_t t = t0 + (tid >> 3) + 32 * p;
            st.pm[p] = t < n ? pre_mix[t * hc + j] : 0.f;
        }
    }
}

// ws: three planes (hi, mid, lo) of 16 R rows each.
template <int R, bool kPre>
__device__ __forceinline__ void stage_store_bf16(const Bf16Stage<R, kPre>& st, uint16_t* xs, uint16_t* ws) {
    const int tid = threadIdx.x, col = (tid & 7) * 8;
#pragma unroll
    for (int p = 0; p < bf16_x_slots(R, kPre); ++p)
        *reinterpret_cast<uint4*>(xs + ((tid >> 3) + 32 * p) * kBRow + col) = st.xw[p];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = (tid >> 4) + 16 * r, lc = (tid & 15) * 4;
        uint32_t h0, m0, l0, h1, m1, l1;
        split3_pair(__uint_as_float(st.wv[r].x), __uint_as_float(st.wv[r].y), h0, m0, l0);
        split3_pair(__uint_as_float(st.wv[r].z), __uint_as_float(st.wv[r].w), h1, m1, l1);
        uint16_t* row = ws + i * kBRow + lc;
        *reinterpret_cast<uint2*>(row) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(row + 16 * R * kBRow) = make_uint2(m0, m1);
        *reinterpret_cast<uint2*>(row + 32 * R * kBRow) = make_uint2(l0, l1);
    }
}

template <int R, bool kPre>
__global__ __launch_bounds__(kGBlock, 2)   // at least two waves per SIMD
void mixes_partial_bf16_kernel(const uint16_t* __restrict__ x, const float* __restrict__ hc_fn, int64_t n, int hc,
                               int64_t d, int blk_per_split, int nsplit, float* __restrict__ part, int pg,
                               const float* __restrict__ pre_mix, uint16_t* __restrict__ y) {
    constexpr int kBT = bf16_row_tiles(R, kPre), kBTok = 64 * kBT, kSlots = bf16_x_slots(R, kPre);
    __shared__ __attribute__((aligned(16))) uint16_t xs[kBTok * kBRow];
    __shared__ __attribute__((aligned(16))) uint16_t ws[3 * 16 * R * kBRow];
    const int M = (2 + hc) * hc;
    const int64_t K = (int64_t)hc * d;
    const int64_t tile = blockIdx.x / nsplit;
    const int slice = (int)(blockIdx.x - tile * nsplit);
    const int64_t t0 = tile * kBTok;
    const int64_t nblk = (d + kGCols - 1) / kGCols;
    const int64_t b_begin = (int64_t)slice * blk_per_split;
    const int64_t b_end = b_begin + blk_per_split < nblk ? b_begin + blk_per_split : nblk;
    const int ntiles = (int)(b_end - b_begin) * hc;   // >= hc: slices are never empty
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    floatx4_g acc[kBT][R], gram[kBT];
#pragma unroll
    for (int T = 0; T < kBT; ++T) {
        gram[T] = floatx4_g{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < R; ++r) acc[T][r] = floatx4_g{0.f, 0.f, 0.f, 0.f};
    }
    float yacc[kPre ? kSlots : 1][8];
#pragma unroll
    for (int p = 0; p < (kPre ? kSlots : 1); ++p)
#pragma unroll
        for (int i = 0; i < 8; ++i) yacc[p][i] = 0.f;
    Bf16Src<R, kPre> src;
    make_src_bf16<R, kPre>(src, x, hc_fn, n, M, K, t0);
    Bf16Stage<R, kPre> st;
    stage_load_bf16<R, kPre>(st, src, pre_mix, n, hc, d, t0, b_begin, 0);
    const uint16_t* xa = xs + (w * 16 * kBT + r16) * kBRow + g * 8;
    const uint16_t* wb = ws + r16 * kBRow + g * 8;
    int64_t b = b_begin;
    int j = 0;
    for (int it = 0; it < ntiles; ++it) {
        __syncthreads();   // the previous tile is consumed
        stage_store_bf16<R, kPre>(st, xs, ws);
        if constexpr (kPre) {
            // collapse: stream j of block b, in ascending j; stored after the last stream
#pragma unroll
            for (int p = 0; p < kSlots; ++p) {
                const uint32_t u[4] = {st.xw[p].x, st.xw[p].y, st.xw[p].z, st.xw[p].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    yacc[p][2 * q] = fmaf(st.pm[p], bf16_lo_g(u[q]), yacc[p][2 * q]);
                    yacc[p][2 * q + 1] = fmaf(st.pm[p], bf16_hi_g(u[q]), yacc[p][2 * q + 1]);
                }
            }
            if (j == hc - 1) {
                const int64_t e = b * kGCols + (tid & 7) * 8;
#pragma unroll
                for (int p = 0; p < kSlots; ++p) {
                    const int64_t t = t0 + (tid >> 3) + 32 * p;
                    if (t < n && e < d)
                        *reinterpret_cast<uint4*>(y + t * d + e) =
                            make_uint4(pack2(yacc[p][0], yacc[p][1]), pack2(yacc[p][2], yacc[p][3]),
                                       pack2(yacc[p][4], yacc[p][5]), pack2(yacc[p][6], yacc[p][7]));
#pragma unroll
                    for (int i = 0; i < 8; ++i) yacc[p][i] = 0.f;
                }
            }
        }
        __syncthreads();
        if (++j == hc) {
            j = 0;
            ++b;
        }
        if (it + 1 < ntiles)   // the next tile's loads run under this tile's MFMAs
            stage_load_bf16<R, kPre>(st, src, pre_mix, n, hc, d, t0, b, j);
#pragma unroll
        for (int kb = 0; kb < kGCols / 32; ++kb) {
            bf16x8_g a[kBT], bv[2][3];
#pragma unroll
            for (int T = 0; T < kBT; ++T)
                a[T] = *reinterpret_cast<const bf16x8_g*>(xa + T * 16 * kBRow + kb * 32);
#pragma unroll
            for (int plane = 0; plane < 3; ++plane)
                bv[0][plane] = *reinterpret_cast<const bf16x8_g*>(wb + plane * 16 * R * kBRow + kb * 32);
            // column tile r + 1's operands are read while tile r is multiplied
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (r + 1 < R) {
#pragma unroll
                    for (int plane = 0; plane < 3; ++plane)
                        bv[(r + 1) & 1][plane] = *reinterpret_cast<const bf16x8_g*>(
                            wb + ((r + 1) * 16 + plane * 16 * R) * kBRow + kb * 32);
                }
#pragma unroll
                for (int plane = 0; plane < 3; ++plane)
#pragma unroll
                    for (int T = 0; T < kBT; ++T)
                        acc[T][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[T], bv[r & 1][plane], acc[T][r], 0,
                                                                            0, 0);
            }
#pragma unroll
            for (int T = 0; T < kBT; ++T)
                gram[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[T], a[T], gram[T], 0, 0, 0);
        }
    }
    // accumulator lane l of row tile T: tokens T*16 + 4 g + i (i < 4) of the wave's, mix r*16 + r16
#pragma unroll
    for (int T = 0; T < kBT; ++T) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int mix = r * 16 + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t t = t0 + w * 16 * kBT + T * 16 + 4 * g + i;
                if (t < n && mix < M) part[((int64_t)slice * n + t) * pg + mix] = acc[T][r][i];
            }
        }
        // the diagonal: lane r16 == 4 g + i holds token T*16 + r16's sum of squares
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + w * 16 * kBT + T * 16 + r16;
            if (r16 == 4 * g + i && t < n) part[((int64_t)slice * n + t) * pg + M] = gram[T][i];
        }
    }
}

// ---------------------------------------- wide projection (bf16, 5 to 8 streams)
// Workgroup (tile, slice): 256 tokens t0 .. t0 + 255 and a slice of 64-channel
// blocks, walked in the tiles of mixes_partial_bf16_kernel (block b of stream 0,
// 1, ..., hc-1, then block b + 1); twelve waves in two roles that meet at one
// barrier per tile, through double-buffered LDS.
//
// Staging (waves 4-11, lane s = tid - 256 of 512): fetches each tile two tiles
// ahead into registers (stream slot p: token row s / 8 + 64 p, channels 8 (s % 8)
// .. +8; weight slot r: row s / 16 + 32 r, columns 4 (s % 16) .. +4), writes the
// stream tile to LDS as it is and the weights split into three bf16 planes, and
// accumulates the collapse (as mixes_partial_bf16_kernel: ascending stream, one
// fma each, stored after the block's last stream).
//
// Multiplying (waves 0-3): wave w takes tokens 64 w .. 64 w + 63 (four row
// tiles) times every mix column tile, with the MFMA steps of
// mixes_partial_bf16_kernel; each weight plane read from LDS serves 64 tokens,
// and a weight tile is fetched and split once per 256 tokens. These waves do
// nothing but LDS reads and MFMAs; the staging work runs on the other eight
// waves, beside them on the same SIMDs.
constexpr int kWTok = 256;        // tokens per workgroup
constexpr int kWThreads = 768;    // 4 multiplying + 8 staging waves
constexpr int kWStage = kWThreads - 256;      // staging lanes
constexpr int kWSlots = kWTok * 8 / kWStage;  // stream slots per staging lane (4)

__host__ __device__ constexpr int wide_lds_bytes(int R) { return 2 * (kWTok + 3 * 16 * R) * kBRow * 2; }
__host__ __device__ constexpr int wide_w_slots(int R) { return (16 * R + 31) / 32; }   // weight slots per lane

template <int R, bool kPre>
struct WideStage {
    uint4 xw[kWSlots];
    uint4 wv[wide_w_slots(R)];
    float pm[kPre ? kWSlots : 1];
};

template <int R>
struct WideSrc {
    __amdgpu_buffer_rsrc_t x[kWSlots];
    __amdgpu_buffer_rsrc_t w[wide_w_slots(R)];
    uint32_t xoff, woff;
};

template <int R, bool kPre>
__device__ __forceinline__ void wide_load(WideStage<R, kPre>& st, const WideSrc<R>& src, const float* pre_mix,
                                          int64_t n, int hc, int64_t d, int64_t t0, int64_t b, int j) {
    const int s = threadIdx.x - 256;
    const int64_t e0 = b * kGCols, c0 = (int64_t)j * d + e0;
    const uint32_t xo = e0 + (s & 7) * 8 < d ? src.xoff : kOffMaskedG;   // d is a multiple of 8
    const uint32_t wo = e0 + (s & 15) * 4 < d ? src.woff : kOffMaskedG;
#pragma unroll
    for (int p = 0; p < kWSlots; ++p) st.xw[p] = bload16(src.x[p], xo, (uint32_t)(c0 * 2));
#pragma unroll
    for (int r = 0; r < wide_w_slots(R); ++r) st.wv[r] = bload16(src.w[r], wo, (uint32_t)(c0 * 4));
    if constexpr (kPre) {
#pragma unroll
        for (int p = 0; p < kWSlots; ++p) {
            const int64_t t = t0 + (s >> 3) + 64 * p;
            st.pm[p] = t < n ? pre_mix[t * hc + j] : 0.f;
        }
    }
}

// Writes tile (b, j) to LDS buffers xs / ws and adds it to the collapse; the
// collapse of block b is stored after its last stream.
template <int R, bool kPre>
__device__ __forceinline__ void wide_store(const WideStage<R, kPre>& st, uint16_t* xs, uint16_t* ws,
                                           float (&yacc)[kPre ? kWSlots : 1][8], uint16_t* __restrict__ y,
                                           int64_t n, int hc, int64_t d, int64_t t0, int64_t b, int j) {
    const int s = threadIdx.x - 256, col = (s & 7) * 8;
#pragma unroll
    for (int p = 0; p < kWSlots; ++p)
        *reinterpret_cast<uint4*>(xs + ((s >> 3) + 64 * p) * kBRow + col) = st.xw[p];
#pragma unroll
    for (int r = 0; r < wide_w_slots(R); ++r) {
        const int i = (s >> 4) + 32 * r, lc = (s & 15) * 4;
        if (16 * R % 32 == 0 || i < 16 * R) {   // the last slot may run past the tile's rows
            uint32_t h0, m0, l0, h1, m1, l1;
            split3_pair(__uint_as_float(st.wv[r].x), __uint_as_float(st.wv[r].y), h0, m0, l0);
            split3_pair(__uint_as_float(st.wv[r].z), __uint_as_float(st.wv[r].w), h1, m1, l1);
            uint16_t* row = ws + i * kBRow + lc;
            *reinterpret_cast<uint2*>(row) = make_uint2(h0, h1);
            *reinterpret_cast<uint2*>(row + 16 * R * kBRow) = make_uint2(m0, m1);
            *reinterpret_cast<uint2*>(row + 32 * R * kBRow) = make_uint2(l0, l1);
        }
    }
    if constexpr (kPre) {
#pragma unroll
        for (int p = 0; p < kWSlots; ++p) {
            const uint32_t u[4] = {st.xw[p].x, st.xw[p].y, st.xw[p].z, st.xw[p].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                yacc[p][2 * q] = fmaf(st.pm[p], bf16_lo_g(u[q]), yacc[p][2 * q]);
                yacc[p][2 * q + 1] = fmaf(st.pm[p], bf16_hi_g(u[q]), yacc[p][2 * q + 1]);
            }
        }
        if (j == hc - 1) {
            const int64_t e = b * kGCols + (s & 7) * 8;
#pragma unroll
            for (int p = 0; p < kWSlots; ++p) {
                const int64_t t = t0 + (s >> 3) + 64 * p;
                if (t < n && e < d)
                    *reinterpret_cast<uint4*>(y + t * d + e) =
                        make_uint4(pack2(yacc[p][0], yacc[p][1]), pack2(yacc[p][2], yacc[p][3]),
                                   pack2(yacc[p][4], yacc[p][5]), pack2(yacc[p][6], yacc[p][7]));
#pragma unroll
                for (int i = 0; i < 8; ++i) yacc[p][i] = 0.f;
            }
        }
    }
}

// Staging role: 1 + ntile barriers, as the multiplying role. Tile u sits in
// register stage u % 2; tiles u + 2 and u + 3 are in flight while tile u is
// multiplied.
template <int R, bool kPre>
__device__ __forceinline__ void wide_stage_role(const uint16_t* __restrict__ x, const float* __restrict__ hc_fn,
                                                const float* __restrict__ pre_mix, int64_t n, int hc, int64_t d,
                                                int64_t t0, int64_t b_begin, int ntile, uint16_t* xs, uint16_t* ws,
                                                uint16_t* __restrict__ y) {
    const int s = threadIdx.x - 256;
    const int M = (2 + hc) * hc;
    const int64_t K = (int64_t)hc * d;
    WideSrc<R> src;
#pragma unroll
    for (int p = 0; p < kWSlots; ++p) {
        const int64_t row0 = t0 + 64 * p;
        src.x[p] = rsrc_g(x + row0 * K, (n - row0) * K * 2);
    }
#pragma unroll
    for (int r = 0; r < wide_w_slots(R); ++r)
        src.w[r] = rsrc_g(hc_fn + (int64_t)32 * r * K, (int64_t)(M - 32 * r) * K * 4);
    src.xoff = (uint32_t)((int64_t)(s >> 3) * K * 2 + (s & 7) * 16);
    src.woff = (uint32_t)((int64_t)(s >> 4) * K * 4 + (s & 15) * 16);
    constexpr int kXBuf = kWTok * kBRow, kWBuf = 3 * 16 * R * kBRow;
    float yacc[kPre ? kWSlots : 1][8];
#pragma unroll
    for (int p = 0; p < (kPre ? kWSlots : 1); ++p)
#pragma unroll
        for (int i = 0; i < 8; ++i) yacc[p][i] = 0.f;
    auto tile_bj = [&](int u, int64_t& b, int& j) {
        const int q = u / hc;
        b = b_begin + q;
        j = u - q * hc;
    };
    WideStage<R, kPre> st[2];
    int64_t b;
    int j;
    tile_bj(0, b, j);
    wide_load<R, kPre>(st[0], src, pre_mix, n, hc, d, t0, b, j);
    if (ntile > 1) {
        tile_bj(1, b, j);
        wide_load<R, kPre>(st[1], src, pre_mix, n, hc, d, t0, b, j);
    }
    tile_bj(0, b, j);
    wide_store<R, kPre>(st[0], xs, ws, yacc, y, n, hc, d, t0, b, j);
    if (ntile > 2) {
        tile_bj(2, b, j);
        wide_load<R, kPre>(st[0], src, pre_mix, n, hc, d, t0, b, j);
    }
    __syncthreads();   // tile 0 is staged
    for (int u0 = 0; u0 < ntile; u0 += 2) {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            const int u = u0 + sl;   // the tile being multiplied; u % 2 == sl
            if (u < ntile) {
                if (u + 1 < ntile) {
                    tile_bj(u + 1, b, j);
                    wide_store<R, kPre>(st[1 - sl], xs + (1 - sl) * kXBuf, ws + (1 - sl) * kWBuf, yacc, y, n, hc,
                                        d, t0, b, j);
                    if (u + 3 < ntile) {
                        tile_bj(u + 3, b, j);
                        wide_load<R, kPre>(st[1 - sl], src, pre_mix, n, hc, d, t0, b, j);
                    }
                }
                __syncthreads();   // tile u is consumed, tile u + 1 is staged
            }
        }
    }
}

template <int R>
__device__ __forceinline__ void wide_mul_role(int64_t n, int hc, int64_t t0, int ntile, int slice, const uint16_t* xs,
                                              const uint16_t* ws, float* __restrict__ part, int pg) {
    constexpr int kBT = 4;
    constexpr int kXBuf = kWTok * kBRow, kWBuf = 3 * 16 * R * kBRow;
    const int M = (2 + hc) * hc;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    floatx4_g acc[kBT][R], gram[kBT];
#pragma unroll
    for (int T = 0; T < kBT; ++T) {
        gram[T] = floatx4_g{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < R; ++r) acc[T][r] = floatx4_g{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();   // tile 0 is staged
    for (int u = 0; u < ntile; ++u) {
        const uint16_t* xa = xs + (u & 1) * kXBuf + (w * 16 * kBT + r16) * kBRow + g * 8;
        const uint16_t* wb = ws + (u & 1) * kWBuf + r16 * kBRow + g * 8;
#pragma unroll
        for (int kb = 0; kb < kGCols / 32; ++kb) {
            bf16x8_g a[kBT], bv[2][3];
#pragma unroll
            for (int T = 0; T < kBT; ++T)
                a[T] = *reinterpret_cast<const bf16x8_g*>(xa + T * 16 * kBRow + kb * 32);
#pragma unroll
            for (int plane = 0; plane < 3; ++plane)
                bv[0][plane] = *reinterpret_cast<const bf16x8_g*>(wb + plane * 16 * R * kBRow + kb * 32);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (r + 1 < R) {
#pragma unroll
                    for (int plane = 0; plane < 3; ++plane)
                        bv[(r + 1) & 1][plane] = *reinterpret_cast<const bf16x8_g*>(
                            wb + ((r + 1) * 16 + plane * 16 * R) * kBRow + kb * 32);
                }
#pragma unroll
                for (int plane = 0; plane < 3; ++plane)
#pragma unroll
                    for (int T = 0; T < kBT; ++T)
                        acc[T][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[T], bv[r & 1][plane], acc[T][r], 0,
                                                                            0, 0);
            }
#pragma unroll
            for (int T = 0; T < kBT; ++T)
                gram[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[T], a[T], gram[T], 0, 0, 0);
        }
        __syncthreads();   // tile u is consumed, tile u + 1 is staged
    }
    // accumulator lane l of row tile T: tokens 64 w + 16 T + 4 g + i, mix 16 r + r16
#pragma unroll
    for (int T = 0; T < kBT; ++T) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int mix = r * 16 + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t t = t0 + w * 16 * kBT + T * 16 + 4 * g + i;
                if (t < n && mix < M) part[((int64_t)slice * n + t) * pg + mix] = acc[T][r][i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + w * 16 * kBT + T * 16 + r16;
            if (r16 == 4 * g + i && t < n) part[((int64_t)slice * n + t) * pg + M] = gram[T][i];
        }
    }
}

template <int R, bool kPre>
__global__ __launch_bounds__(kWThreads, 1)
void mixes_wide_bf16_kernel(const uint16_t* __restrict__ x, const float* __restrict__ hc_fn, int64_t n, int hc,
                            int64_t d, int blk_per_split, int nsplit, float* __restrict__ part, int pg,
                            const float* __restrict__ pre_mix, uint16_t* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[2 * kWTok * kBRow];
    __shared__ __attribute__((aligned(16))) uint16_t ws[2 * 3 * 16 * R * kBRow];
    const int64_t tile = blockIdx.x / nsplit;
    const int slice = (int)(blockIdx.x - tile * nsplit);
    const int64_t t0 = tile * kWTok;
    const int64_t nblk = (d + kGCols - 1) / kGCols;
    const int64_t b_begin = (int64_t)slice * blk_per_split;
    const int64_t b_end = b_begin + blk_per_split < nblk ? b_begin + blk_per_split : nblk;
    const int ntile = (int)(b_end - b_begin) * hc;   // >= hc: slices are never empty
    if (__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) >= 4)   // wave-uniform role
        wide_stage_role<R, kPre>(x, hc_fn, pre_mix, n, hc, d, t0, b_begin, ntile, xs, ws, y);
    else
        wide_mul_role<R>(n, hc, t0, ntile, slice, xs, ws, part, pg);
}

// A wave per token: lane l sums entries l and l + 64 of the partial rows over the
// slices in order, then scales the dots by 1 / sqrt(sum of squares / (hc d) + eps).
// Token t's mixes from its partial rows: lane l gets mixes l (a0) and l + 64 (a1),
// already scaled; stores them when `mixes` is not null.
__device__ __forceinline__ void finalize_mixes_wave(const float* __restrict__ part, int nsplit, int pg, int64_t n,
                                                    int hc, int64_t d, float norm_eps, float* __restrict__ mixes,
                                                    int64_t t, float& m0, float& m1) {
    const int lane = threadIdx.x & 63;
    const int M = (2 + hc) * hc;
    const int i0 = lane, i1 = lane + 64;
    float a0 = 0.f, a1 = 0.f;
    // 16 slices' loads are issued before they are added (in slice order; a
    // missing slice adds +0)
    for (int s0 = 0; s0 < nsplit; s0 += 16) {
        float v0[16], v1[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float* row = part + ((int64_t)(s0 + i) * n + t) * pg;
            const bool ok = s0 + i < nsplit;
            v0[i] = ok && i0 <= M ? row[i0] : 0.f;
            v1[i] = ok && i1 <= M ? row[i1] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            a0 += v0[i];
            a1 += v1[i];
        }
    }
    const float ss = M < 64 ? __shfl(a0, M) : __shfl(a1, M - 64);
    const float rstd = 1.0f / sqrtf(ss / (float)((int64_t)hc * d) + norm_eps);
    m0 = a0 * rstd;
    m1 = a1 * rstd;
    if (mixes && i0 < M) mixes[t * M + i0] = m0;
    if (mixes && i1 < M) mixes[t * M + i1] = m1;
}

__global__ __launch_bounds__(kGBlock) void mixes_finalize_kernel(const float* __restrict__ part, int nsplit,
                                                                 int pg, int64_t n, int hc, int64_t d,
                                                                 float norm_eps, float* __restrict__ mixes) {
    const int64_t t = (int64_t)blockIdx.x * (kGBlock / 64) + (threadIdx.x >> 6);
    if (t >= n) return;   // a whole wave leaves together
    float m0, m1;
    finalize_mixes_wave(part, nsplit, pg, n, hc, d, norm_eps, mixes, t, m0, m1);
}

// The finalize and the split in one launch: the split takes the token's mixes
// from the finalizing wave's registers (the same fp32 values the two-kernel path
// stores and reloads). kH = 2 or 8: butterfly sums; 0: any stream count.
template <int kH>
__global__ __launch_bounds__(kGBlock) void finalize_split_kernel(const float* __restrict__ part, int nsplit, int pg,
                                                                 int64_t n, int hc, int64_t d, float norm_eps,
                                                                 float* __restrict__ mixes,
                                                                 const float* __restrict__ scale,
                                                                 const float* __restrict__ base, int iters, float eps,
                                                                 float* __restrict__ pre, float* __restrict__ post,
                                                                 float* __restrict__ comb) {
    const int64_t t = (int64_t)blockIdx.x * (kGBlock / 64) + (threadIdx.x >> 6);
    if (t >= n) return;   // a whole wave leaves together
    float m0, m1;
    finalize_mixes_wave(part, nsplit, pg, n, hc, d, norm_eps, mixes, t, m0, m1);
    auto mix = [&](int i) {   // every lane calls it: both shuffles run in all lanes
        const float lo = __shfl(m0, i & 63), hi = __shfl(m1, i & 63);
        return i < 64 ? lo : hi;
    };
    if constexpr (kH == 0)
        split_generic_wave(mix, scale, base, t, hc, iters, eps, pre, post, comb);
    else
        split_butterfly_wave<kH>(mix, scale, base, t, iters, eps, pre, post, comb);
}

// Two streams: the finalize and the split with 4 lanes per token (16 tokens per
// wave; a wave per token left 60 of its 64 lanes idle through the Sinkhorn
// rounds). Lane q < 3 of a token's quad sums float4 q of its partial rows (12
// floats: dots 0..7, the sum of squares at 8) over the slices in order; slices
// past nsplit and lane 3 re-read a valid row and add zero instead. Every lane of
// the quad then takes lanes 0 and 1's sums (mixes 0..3: pre and post logits,
// 4..7: the 2 x 2 comb) and runs the same steps as split_butterfly_wave<2> in
// registers, where a row or column sum is one add of the same two numbers (as in
// the butterfly, both without contraction), so the results are the same bits;
// lane 0 stores pre, lane 1 post, lane 2 the comb. Lanes past n compute on token
// n - 1 and store nothing.
constexpr int kF2Pg = 12;
static_assert((((2 + 2) * 2 + 1 + 3) & ~3) == kF2Pg, "the plan's partial-row pitch at two streams");
__global__ __launch_bounds__(kGBlock) void finalize_split2_kernel(const float* __restrict__ part, int nsplit,
                                                                  int64_t n, int64_t d, float norm_eps,
                                                                  float* __restrict__ mixes,
                                                                  const float* __restrict__ scale,
                                                                  const float* __restrict__ base, int iters,
                                                                  float eps, float* __restrict__ pre,
                                                                  float* __restrict__ post, float* __restrict__ comb) {
    // No contraction here: in registers the compiler would fuse a product into the
    // next row or column sum, which the butterfly (whose sums read other lanes)
    // cannot; the fused multiply-adds the butterfly does get are written out.
#pragma clang fp contract(off)
    const int q = threadIdx.x & 3;
    const int64_t t = ((int64_t)blockIdx.x * kGBlock + threadIdx.x) >> 2;
    const bool ok = t < n;
    const int64_t tt = ok ? t : n - 1;
    const int qc = q < 3 ? q : 2;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < nsplit; s0 += 16) {
        float4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int sc = s0 + i < nsplit ? s0 + i : nsplit - 1;
            v[i] = *reinterpret_cast<const float4*>(part + ((int64_t)sc * n + tt) * kF2Pg + 4 * qc);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const bool keep = s0 + i < nsplit && q < 3;
            acc.x += keep ? v[i].x : 0.f;
            acc.y += keep ? v[i].y : 0.f;
            acc.z += keep ? v[i].z : 0.f;
            acc.w += keep ? v[i].w : 0.f;
        }
    }
    constexpr int kBcast0 = 0x00, kBcast1 = 0x55, kBcast2 = 0xAA;   // quad_perm: every lane reads lane 0 / 1 / 2
    const float ss = dpp_g<kBcast2>(acc.x);
    const float rstd = 1.0f / sqrtf(ss / (float)(2 * d) + norm_eps);
    const float4 lo = make_float4(dpp_g<kBcast0>(acc.x) * rstd, dpp_g<kBcast0>(acc.y) * rstd,
                                  dpp_g<kBcast0>(acc.z) * rstd, dpp_g<kBcast0>(acc.w) * rstd);
    const float4 cm = make_float4(dpp_g<kBcast1>(acc.x) * rstd, dpp_g<kBcast1>(acc.y) * rstd,
                                  dpp_g<kBcast1>(acc.z) * rstd, dpp_g<kBcast1>(acc.w) * rstd);
    if (mixes && ok && q < 2)
        reinterpret_cast<float4*>(mixes)[t * 2 + q] = make_float4(q == 0 ? lo.x : cm.x, q == 0 ? lo.y : cm.y,
                                                                  q == 0 ? lo.z : cm.z, q == 0 ? lo.w : cm.w);
    // comb logits C[j][k] = mixes[4 + 2 j + k]
    float c00 = fmaf(cm.x, scale[2], base[4]), c01 = fmaf(cm.y, scale[2], base[5]);
    float c10 = fmaf(cm.z, scale[2], base[6]), c11 = fmaf(cm.w, scale[2], base[7]);
    const float m0 = fmaxf(c00, c01), m1 = fmaxf(c10, c11);
    c00 = __expf(c00 - m0); c01 = __expf(c01 - m0);
    c10 = __expf(c10 - m1); c11 = __expf(c11 - m1);
    float r0 = __builtin_amdgcn_rcpf(c00 + c01), r1 = __builtin_amdgcn_rcpf(c10 + c11);
    c00 = fmaf(c00, r0, eps); c01 = fmaf(c01, r0, eps);
    c10 = fmaf(c10, r1, eps); c11 = fmaf(c11, r1, eps);
    float k0 = __builtin_amdgcn_rcpf(c00 + c10 + eps), k1 = __builtin_amdgcn_rcpf(c01 + c11 + eps);
    c00 *= k0; c10 *= k0; c01 *= k1; c11 *= k1;
    for (int it = 1; it < iters; ++it) {
        r0 = __builtin_amdgcn_rcpf(c00 + c01 + eps);
        r1 = __builtin_amdgcn_rcpf(c10 + c11 + eps);
        c00 *= r0; c01 *= r0; c10 *= r1; c11 *= r1;
        k0 = __builtin_amdgcn_rcpf(c00 + c10 + eps);
        k1 = __builtin_amdgcn_rcpf(c01 + c11 + eps);
        c00 *= k0; c10 *= k0; c01 *= k1; c11 *= k1;
    }
    if (!ok) return;
    if (q == 0)
        reinterpret_cast<float2*>(pre)[t] = make_float2(sigmoid_f(fmaf(lo.x, scale[0], base[0])) + eps,
                                                        sigmoid_f(fmaf(lo.y, scale[0], base[1])) + eps);
    else if (q == 1)
        reinterpret_cast<float2*>(post)[t] = make_float2(2.0f * sigmoid_f(fmaf(lo.z, scale[1], base[2])),
                                                         2.0f * sigmoid_f(fmaf(lo.w, scale[1], base[3])));
    else if (q == 2)
        reinterpret_cast<float4*>(comb)[t] = make_float4(c00, c01, c10, c11);
}

int64_t ceil_div_g(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct GenericPlan {
    int64_t tiles;
    int per_split;      // flattened columns (fp32 plan) or 64-channel blocks (bf16 plan) per slice
    int nsplit;
    int pg;             // floats per partial row: (2+hc)hc dots + the sum of squares, padded to 4
    size_t mixes_offset;  // scratch mixes after the partial rows (fused step)
    size_t total_bytes;
};

int64_t slice_count(int64_t tiles, int64_t units) {
    int64_t ns = ceil_div_g(512, tiles > 0 ? tiles : 1);   // about two workgroups per CU
    if (ns > units) ns = units;
    if (ns > kGMaxSplit) ns = kGMaxSplit;
    return ns < 1 ? 1 : ns;
}

// fp32 streams: 64-token tiles x slices of whole 64-column tiles of the flattened axis.
GenericPlan plan_f32(int64_t n, int hc, int64_t d) {
    GenericPlan p{};
    const int64_t K = (int64_t)hc * d, ncols = ceil_div_g(K, kGCols);
    p.tiles = ceil_div_g(n, kGTok);
    p.per_split = (int)(ceil_div_g(ncols, slice_count(p.tiles, ncols)) * kGCols);
    p.nsplit = (int)ceil_div_g(K, p.per_split);
    return p;
}

// bf16 streams: 64 kBT-token tiles x slices of 64-channel blocks (all streams).
GenericPlan plan_bf16(int64_t n, int hc, int64_t d, bool pre) {
    GenericPlan p{};
    const int M = (2 + hc) * hc;
    const int64_t nblk = ceil_div_g(d, kGCols);
    p.tiles = ceil_div_g(n, 64 * bf16_row_tiles((M + 15) / 16, pre));
    p.per_split = (int)ceil_div_g(nblk, slice_count(p.tiles, nblk));
    p.nsplit = (int)ceil_div_g(nblk, p.per_split);
    return p;
}

// bf16 streams, five to eight (wide kernel): 256-token tiles x slices of 64-channel
// blocks, one workgroup per CU (its LDS), 256 CUs.
bool use_wide(int hc) { return hc >= 5; }

GenericPlan plan_wide(int64_t n, int64_t d) {
    GenericPlan p{};
    const int64_t nblk = ceil_div_g(d, kGCols);
    p.tiles = ceil_div_g(n, kWTok);
    int64_t ns = ceil_div_g(256, p.tiles);
    if (ns > nblk) ns = nblk;
    if (ns > kGMaxSplit) ns = kGMaxSplit;
    if (ns < 1) ns = 1;
    p.per_split = (int)ceil_div_g(nblk, ns);
    p.nsplit = (int)ceil_div_g(nblk, p.per_split);
    return p;
}

// The workspace layout does not depend on the stream dtype or on the collapse:
// room for the partial rows of the largest plan, then the scratch mixes.
GenericPlan plan_generic(int64_t n, int hc, int64_t d, bool bf16, bool pre) {
    GenericPlan p = bf16 ? (use_wide(hc) ? plan_wide(n, d) : plan_bf16(n, hc, d, pre)) : plan_f32(n, hc, d);
    const int M = (2 + hc) * hc;
    p.pg = (M + 1 + 3) & ~3;
    int ns_max = plan_f32(n, hc, d).nsplit;
    for (int q = 0; q < 2; ++q) {
        const int ns = plan_bf16(n, hc, d, q == 1).nsplit;
        if (ns > ns_max) ns_max = ns;
    }
    if (use_wide(hc) && plan_wide(n, d).nsplit > ns_max) ns_max = plan_wide(n, d).nsplit;
    p.mixes_offset = ((size_t)ns_max * (size_t)n * (size_t)p.pg * sizeof(float) + 255) & ~size_t(255);
    p.total_bytes = p.mixes_offset + (size_t)n * (size_t)M * sizeof(float);
    return p;
}

void launch_partial_f32(const GenericPlan& p, const void* xv, const float* hc_fn, int64_t n, int hc, int64_t d,
                        float* part, hipStream_t stream) {
    const int M = (2 + hc) * hc;
    const float* x = static_cast<const float*>(xv);
    const dim3 grid((unsigned)(p.tiles * p.nsplit)), block(kGBlock);
    switch ((M + 15) / 16) {
        case 1: hipLaunchKernelGGL((mixes_partial_kernel<1>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                   p.per_split, p.nsplit, part, p.pg); break;
        case 2: hipLaunchKernelGGL((mixes_partial_kernel<2>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                   p.per_split, p.nsplit, part, p.pg); break;
        case 3: hipLaunchKernelGGL((mixes_partial_kernel<3>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                   p.per_split, p.nsplit, part, p.pg); break;
        case 4: hipLaunchKernelGGL((mixes_partial_kernel<4>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                   p.per_split, p.nsplit, part, p.pg); break;
        default: hipLaunchKernelGGL((mixes_partial_kernel<5>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                    p.per_split, p.nsplit, part, p.pg); break;
    }
}

template <bool kPre>
void launch_partial_bf16_t(const GenericPlan& p, const uint16_t* x, const float* hc_fn, int64_t n, int hc,
                           int64_t d, float* part, const float* pre_mix, uint16_t* y, hipStream_t stream) {
    const int M = (2 + hc) * hc;
    const dim3 grid((unsigned)(p.tiles * p.nsplit)), block(kGBlock);
    switch ((M + 15) / 16) {
        case 1: hipLaunchKernelGGL((mixes_partial_bf16_kernel<1, kPre>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                   p.per_split, p.nsplit, part, p.pg, pre_mix, y); break;
        case 2: hipLaunchKernelGGL((mixes_partial_bf16_kernel<2, kPre>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                   p.per_split, p.nsplit, part, p.pg, pre_mix, y); break;
        case 3: hipLaunchKernelGGL((mixes_partial_bf16_kernel<3, kPre>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                   p.per_split, p.nsplit, part, p.pg, pre_mix, y); break;
        case 4: hipLaunchKernelGGL((mixes_partial_bf16_kernel<4, kPre>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                   p.per_split, p.nsplit, part, p.pg, pre_mix, y); break;
        default: hipLaunchKernelGGL((mixes_partial_bf16_kernel<5, kPre>), grid, block, 0, stream, x, hc_fn, n, hc,
                                    d, p.per_split, p.nsplit, part, p.pg, pre_mix, y); break;
    }
}

template <int R, bool kPre>
void launch_wide_v(const GenericPlan& p, const uint16_t* x, const float* hc_fn, int64_t n, int hc, int64_t d,
                   float* part, const float* pre_mix, uint16_t* y, hipStream_t stream) {
    static_assert(wide_lds_bytes(R) <= 160 * 1024, "LDS of one CU");
    hipLaunchKernelGGL((mixes_wide_bf16_kernel<R, kPre>), dim3((unsigned)(p.tiles * p.nsplit)), dim3(kWThreads), 0,
                       stream, x, hc_fn, n, hc, d, p.per_split, p.nsplit, part, p.pg, pre_mix, y);
}

template <bool kPre>
void launch_wide(const GenericPlan& p, const uint16_t* x, const float* hc_fn, int64_t n, int hc, int64_t d,
                 float* part, const float* pre_mix, uint16_t* y, hipStream_t stream) {
    switch ((2 + hc) * hc) {
        case 80: launch_wide_v<5, kPre>(p, x, hc_fn, n, hc, d, part, pre_mix, y, stream); break;   // hc = 8
        case 63: launch_wide_v<4, kPre>(p, x, hc_fn, n, hc, d, part, pre_mix, y, stream); break;   // hc = 7
        default: launch_wide_v<3, kPre>(p, x, hc_fn, n, hc, d, part, pre_mix, y, stream); break;   // hc = 5, 6
    }
}

// The projection's partial rows (with the collapse when y is given), then the
// finalize into `mixes`.
struct SplitArgs {   // the split fused into the finalize launch
    const float* scale;
    const float* base;
    int iters;
    float eps;
    float* pre;
    float* post;
    float* comb;
};

// Projection partials, then the finalize (and, when `sp` is given, the split in the
// same launch; `mixes` may then be null).
hipError_t launch_projection(const void* x, bool bf16, int64_t n, int hc, int64_t d, const float* hc_fn,
                             float norm_eps, float* mixes, void* workspace, const float* pre_mix, void* y,
                             hipStream_t stream, const SplitArgs* sp = nullptr) {
    const GenericPlan p = plan_generic(n, hc, d, bf16, y != nullptr);
    float* part = static_cast<float*>(workspace);
    if (bf16 && use_wide(hc)) {
        const uint16_t* xb = static_cast<const uint16_t*>(x);
        if (y)
            launch_wide<true>(p, xb, hc_fn, n, hc, d, part, pre_mix, static_cast<uint16_t*>(y), stream);
        else
            launch_wide<false>(p, xb, hc_fn, n, hc, d, part, nullptr, nullptr, stream);
    } else if (bf16) {
        const uint16_t* xb = static_cast<const uint16_t*>(x);
        if (y)
            launch_partial_bf16_t<true>(p, xb, hc_fn, n, hc, d, part, pre_mix, static_cast<uint16_t*>(y), stream);
        else
            launch_partial_bf16_t<false>(p, xb, hc_fn, n, hc, d, part, nullptr, nullptr, stream);
    } else {
        launch_partial_f32(p, x, hc_fn, n, hc, d, part, stream);
    }
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const dim3 grid((unsigned)ceil_div_g(n, kGBlock / 64));
    if (!sp)
        hipLaunchKernelGGL(mixes_finalize_kernel, grid, dim3(kGBlock), 0, stream, part, p.nsplit, p.pg, n, hc, d,
                           norm_eps, mixes);
    else if (hc == 8)
        hipLaunchKernelGGL(finalize_split_kernel<8>, grid, dim3(kGBlock), 0, stream, part, p.nsplit, p.pg, n, hc, d,
                           norm_eps, mixes, sp->scale, sp->base, sp->iters, sp->eps, sp->pre, sp->post, sp->comb);
    else if (hc == 2)
        hipLaunchKernelGGL(finalize_split2_kernel, dim3((unsigned)ceil_div_g(n, kGBlock / 4)), dim3(kGBlock), 0,
                           stream, part, p.nsplit, n, d, norm_eps, mixes, sp->scale, sp->base, sp->iters, sp->eps,
                           sp->pre, sp->post, sp->comb);
    else
        hipLaunchKernelGGL(finalize_split_kernel<0>, grid, dim3(kGBlock), 0, stream, part, p.nsplit, p.pg, n, hc, d,
                           norm_eps, mixes, sp->scale, sp->base, sp->iters, sp->eps, sp->pre, sp->post, sp->comb);
    return hipGetLastError();
}

}  // namespace

// Work-items of the largest grid the launchers of this file form for (n, hc, d):
// the projection (both stream dtypes, with and without the collapse), the
// finalize and split (a wave per token), and the collapse and expand (a wave per
// token and 512 channels).
int64_t generic_max_launch_items(int64_t n, int hc, int64_t d) {
    int64_t m = ceil_div_g(n, kGBlock / 64) * kGBlock;
    const int64_t ew = wave_grid(n, d) * kGBlock;
    if (ew > m) m = ew;
    const GenericPlan plans[] = {plan_f32(n, hc, d), plan_bf16(n, hc, d, false), plan_bf16(n, hc, d, true)};
    for (const GenericPlan& p : plans)
        if (p.tiles * p.nsplit * kGBlock > m) m = p.tiles * p.nsplit * kGBlock;
    if (use_wide(hc)) {
        const GenericPlan p = plan_wide(n, d);
        if (p.tiles * p.nsplit * kWThreads > m) m = p.tiles * p.nsplit * kWThreads;
    }
    return m;
}

size_t generic_workspace_bytes(int64_t n, int hc, int64_t d) {
    return plan_generic(n, hc, d, true, true).total_bytes;
}

hipError_t launch_split_generic(const float* mixes, const float* scale, const float* base, int64_t n, int hc,
                                int iters, float eps, float* pre, float* post, float* comb, hipStream_t stream) {
    const dim3 grid((unsigned)ceil_div_g(n, kGBlock / 64));
    if (hc == 8)
        hipLaunchKernelGGL(split_butterfly_kernel<8>, grid, dim3(kGBlock), 0, stream, mixes, scale, base, n, iters,
                           eps, pre, post, comb);
    else if (hc == 2)
        hipLaunchKernelGGL(split_butterfly_kernel<2>, grid, dim3(kGBlock), 0, stream, mixes, scale, base, n, iters,
                           eps, pre, post, comb);
    else
        hipLaunchKernelGGL(split_generic_kernel, grid, dim3(kGBlock), 0, stream, mixes, scale, base, n, hc, iters,
                           eps, pre, post, comb);
    return hipGetLastError();
}

hipError_t launch_pre_generic(const void* x, bool bf16, const float* pre_mix, int64_t n, int hc, int64_t d, void* y,
                              hipStream_t stream) {
    const dim3 grid((unsigned)wave_grid(n, d));
    if (bf16)
        hipLaunchKernelGGL(pre_generic_kernel<true>, grid, dim3(kGBlock), 0, stream, x, pre_mix, n, hc, d, y);
    else
        hipLaunchKernelGGL(pre_generic_kernel<false>, grid, dim3(kGBlock), 0, stream, x, pre_mix, n, hc, d, y);
    return hipGetLastError();
}

template <bool kBf16, bool kStream>
void launch_post_generic_v(dim3 grid, const void* f, const void* res, const float* post, const float* comb, int64_t n,
                           int hc, int64_t d, void* out, const float* pre_mix, void* y, hipStream_t stream) {
    if (y)
        hipLaunchKernelGGL((post_generic_kernel<kBf16, kStream, true>), grid, dim3(kGBlock), 0, stream, f, res, post,
                           comb, n, hc, d, out, pre_mix, y);
    else
        hipLaunchKernelGGL((post_generic_kernel<kBf16, kStream, false>), grid, dim3(kGBlock), 0, stream, f, res, post,
                           comb, n, hc, d, out, nullptr, nullptr);
}

// y not null: also the collapse of the new streams with pre_mix into y.
hipError_t launch_post_collapse_generic(const void* f, const void* res, bool bf16, const float* post,
                                        const float* comb, int64_t n, int hc, int64_t d, void* out, hipStream_t stream,
                                        bool stream_out, const float* pre_mix, void* y) {
    const dim3 grid((unsigned)wave_grid(n, d));
    if (bf16 && stream_out)
        launch_post_generic_v<true, true>(grid, f, res, post, comb, n, hc, d, out, pre_mix, y, stream);
    else if (bf16)
        launch_post_generic_v<true, false>(grid, f, res, post, comb, n, hc, d, out, pre_mix, y, stream);
    else if (stream_out)
        launch_post_generic_v<false, true>(grid, f, res, post, comb, n, hc, d, out, pre_mix, y, stream);
    else
        launch_post_generic_v<false, false>(grid, f, res, post, comb, n, hc, d, out, pre_mix, y, stream);
    return hipGetLastError();
}

hipError_t launch_post_generic(const void* f, const void* res, bool bf16, const float* post, const float* comb,
                               int64_t n, int hc, int64_t d, void* out, hipStream_t stream, bool stream_out) {
    return launch_post_collapse_generic(f, res, bf16, post, comb, n, hc, d, out, stream, stream_out, nullptr,
                                        nullptr);
}

hipError_t launch_mixes_generic(const void* x, bool bf16, int64_t n, int hc, int64_t d, const float* hc_fn,
                                float norm_eps, float* mixes, void* workspace, hipStream_t stream) {
    return launch_projection(x, bf16, n, hc, d, hc_fn, norm_eps, mixes, workspace, nullptr, nullptr, stream);
}

// expand (if any) -> projection (with the collapse fused for bf16 streams) ->
// finalize + split (one launch) -> collapse (fp32 streams)
// The expand output that the projection reads next stays cached unless it is
// larger than the 256 MB last-level cache: then the projection cannot find it
// there anyway, and non-temporal stores keep its write-back out of the reads
// (prefill block at 8 streams: 495 -> 482 us; at 2 streams, 84 MB, cached stores
// win: 134 against 139 us).
constexpr int64_t kLastLevelCacheBytes = int64_t(256) << 20;

hipError_t launch_fused_generic(const GenericRequest& r, hipStream_t stream) {
    // With an expand, the expand kernel also collapses the new streams (it holds
    // every stream of its channels); otherwise bf16 streams are collapsed inside
    // the projection and fp32 streams by a collapse kernel after it.
    const bool fused_pre = r.bf16 && r.y && !r.f_prev;
    const SplitArgs sp{r.scale, r.base, r.iters, r.eps, r.pre, r.post, r.comb};
    const void* src = r.res;
    if (r.f_prev) {
        const int64_t out_bytes = r.n * r.hc * r.d * (r.bf16 ? 2 : 4);
        if (hipError_t e = launch_post_collapse_generic(r.f_prev, r.res, r.bf16, r.post_prev, r.comb_prev, r.n, r.hc,
                                                        r.d, r.streams_out, stream, out_bytes > kLastLevelCacheBytes,
                                                        r.y ? r.pre_mix : nullptr, r.y);
            e != hipSuccess)
            return e;
        src = r.streams_out;
    }
    // the finalize splits the mixes in the same launch; they are stored only when asked for
    if (hipError_t e = launch_projection(src, r.bf16, r.n, r.hc, r.d, r.hc_fn, r.norm_eps, r.mixes, r.workspace,
                                         fused_pre ? r.pre_mix : nullptr, fused_pre ? r.y : nullptr, stream, &sp);
        e != hipSuccess)
        return e;
    if (r.y && !fused_pre && !r.f_prev) return launch_pre_generic(src, r.bf16, r.pre_mix, r.n, r.hc, r.d, r.y, stream);
    return hipSuccess;
}

}  // namespace hc
