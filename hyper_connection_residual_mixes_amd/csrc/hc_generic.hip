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
//                           and columns are summed with cross-lane reads.
//   pre_generic_kernel      collapse, one lane per (token, 8 channels).
//   post_generic_kernel     expand + combine, one lane per (token, 8 channels).
//   mixes_partial_kernel    16 tokens x one slice of the flattened hc*d axis per
//                           workgroup: the (2+hc)*hc partial dot products and the
//                           partial sum of squares, from LDS tiles of 64 columns.
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
constexpr int kGTok = 16;       // tokens per projection workgroup
constexpr int kGCols = 64;      // flattened columns per LDS tile
constexpr int kGMaxSplit = 64;  // slices of the flattened axis

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

// Stores eight fp32 values rounded once to the element type.
template <bool kBf16>
__device__ __forceinline__ void store8(void* base, int64_t idx, const float (&v)[8]) {
    if constexpr (kBf16) {
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx) =
            make_uint4(pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7]));
    } else {
        float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + idx);
        p[0] = make_float4(v[0], v[1], v[2], v[3]);
        p[1] = make_float4(v[4], v[5], v[6], v[7]);
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

__global__ __launch_bounds__(kGBlock) void split_generic_kernel(const float* __restrict__ mixes,
                                                                const float* __restrict__ scale,
                                                                const float* __restrict__ base, int64_t n,
                                                                int hc, int iters, float eps,
                                                                float* __restrict__ pre, float* __restrict__ post,
                                                                float* __restrict__ comb) {
    const int64_t t = (int64_t)blockIdx.x * (kGBlock / 64) + (threadIdx.x >> 6);
    if (t >= n) return;   // a whole wave leaves together
    const int lane = threadIdx.x & 63;
    const int M = (2 + hc) * hc, hc2 = hc * hc;
    const float* m = mixes + t * M;
    const bool cl = lane < hc2;
    const int j = cl ? lane / hc : 0;
    const int k = cl ? lane - j * hc : 0;
    const int ci = 2 * hc + (cl ? lane : 0);
    float c = m[ci] * scale[2] + base[ci];
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
        pre[t * hc + lane] = sigmoid_f(m[lane] * scale[0] + base[lane]) + eps;
    else if (lane < 2 * hc)
        post[t * hc + lane - hc] = 2.0f * sigmoid_f(m[lane] * scale[1] + base[lane]);
}

// --------------------------------------------------------- collapse / expand
template <bool kBf16>
__global__ __launch_bounds__(kGBlock) void pre_generic_kernel(const void* __restrict__ x,
                                                              const float* __restrict__ pre_mix, int64_t n,
                                                              int hc, int64_t d, void* __restrict__ y) {
    const int64_t per_tok = d >> 3;
    const int64_t gid = (int64_t)blockIdx.x * kGBlock + threadIdx.x;
    if (gid >= n * per_tok) return;
    const int64_t t = gid / per_tok;
    const int64_t e = (gid - t * per_tok) << 3;
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

// Every stream of the lane's 8 channels is read before any is written, so the
// output may be the residual itself.
template <bool kBf16>
__global__ __launch_bounds__(kGBlock) void post_generic_kernel(const void* __restrict__ f, const void* res,
                                                               const float* __restrict__ post,
                                                               const float* __restrict__ comb, int64_t n, int hc,
                                                               int64_t d, void* out) {
    const int64_t per_tok = d >> 3;
    const int64_t gid = (int64_t)blockIdx.x * kGBlock + threadIdx.x;
    if (gid >= n * per_tok) return;
    const int64_t t = gid / per_tok;
    const int64_t e = (gid - t * per_tok) << 3;
    float fv[8], rv[kMaxHC][8];
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
        store8<kBf16>(out, (t * hc + k) * d + e, o);
    }
}

// ------------------------------------------------------------- projection
// Workgroup (tile, slice): tokens tile*16 .. +16 and flattened columns
// [slice * cols_per_split, +cols_per_split). Lane (tok = tid % 16, g = tid / 16)
// accumulates mix rows g, g + 16, ... (R of them) for its token, and every lane
// the token's sum of squares (the g == 0 lanes store it). Tiles of 64 columns of
// the streams and of hc_fn are staged in LDS (rows padded by one float); rows of
// the hc_fn tile past the last mix stay zero.
template <bool kBf16, int R>
__global__ __launch_bounds__(kGBlock) void mixes_partial_kernel(const void* __restrict__ x,
                                                                const float* __restrict__ hc_fn, int64_t n,
                                                                int hc, int64_t d, int cols_per_split,
                                                                int nsplit, float* __restrict__ part, int pg) {
    __shared__ float xs[kGTok][kGCols + 1];
    __shared__ float ws[16 * R][kGCols + 1];
    const int M = (2 + hc) * hc;
    const int64_t K = (int64_t)hc * d;
    const int64_t tile = blockIdx.x / nsplit;
    const int slice = (int)(blockIdx.x - tile * nsplit);
    const int64_t t0 = tile * kGTok;
    const int64_t c_begin = (int64_t)slice * cols_per_split;
    const int64_t c_end = c_begin + cols_per_split < K ? c_begin + cols_per_split : K;
    const int tid = threadIdx.x, tok = tid % kGTok, g = tid / kGTok;
    for (int q = tid; q < 16 * R * (kGCols + 1); q += kGBlock) (&ws[0][0])[q] = 0.f;
    float acc[R], ss = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
    for (int64_t c0 = c_begin; c0 < c_end; c0 += kGCols) {
        __syncthreads();   // the previous tile is consumed (and the zero fill is done)
        {   // streams: 16 tokens x 64 columns, 4 consecutive columns per lane
            const int lt = tid / 16, lc = (tid % 16) * 4;
            const int64_t t = t0 + lt, c = c0 + lc;
            float v[4] = {0.f, 0.f, 0.f, 0.f};
            if (t < n && c < c_end) {   // K is a multiple of 8: the 4 columns are all in or all out
                if constexpr (kBf16) {
                    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + t * K + c);
                    v[0] = __uint_as_float(w.x << 16);
                    v[1] = __uint_as_float(w.x & 0xffff0000u);
                    v[2] = __uint_as_float(w.y << 16);
                    v[3] = __uint_as_float(w.y & 0xffff0000u);
                } else {
                    const float4 w = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + t * K + c);
                    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) xs[lt][lc + i] = v[i];
        }
        for (int q = tid; q < M * (kGCols / 4); q += kGBlock) {   // hc_fn: M rows x 64 columns
            const int i = q / (kGCols / 4), lc = (q % (kGCols / 4)) * 4;
            const int64_t c = c0 + lc;
            float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < c_end) w = *reinterpret_cast<const float4*>(hc_fn + (int64_t)i * K + c);
            ws[i][lc] = w.x; ws[i][lc + 1] = w.y; ws[i][lc + 2] = w.z; ws[i][lc + 3] = w.w;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < kGCols; ++kk) {
            const float xv = xs[tok][kk];
            ss = fmaf(xv, xv, ss);
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = fmaf(xv, ws[g + 16 * r][kk], acc[r]);
        }
    }
    const int64_t t = t0 + tok;
    if (t >= n) return;
    float* row = part + ((int64_t)slice * n + t) * pg;
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (g + 16 * r < M) row[g + 16 * r] = acc[r];
    if (g == 0) row[M] = ss;
}

// A wave per token: lane l sums entries l and l + 64 of the partial rows over the
// slices in order, then scales the dots by 1 / sqrt(sum of squares / (hc d) + eps).
__global__ __launch_bounds__(kGBlock) void mixes_finalize_kernel(const float* __restrict__ part, int nsplit,
                                                                 int pg, int64_t n, int hc, int64_t d,
                                                                 float norm_eps, float* __restrict__ mixes) {
    const int64_t t = (int64_t)blockIdx.x * (kGBlock / 64) + (threadIdx.x >> 6);
    if (t >= n) return;   // a whole wave leaves together
    const int lane = threadIdx.x & 63;
    const int M = (2 + hc) * hc;
    const int i0 = lane, i1 = lane + 64;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) {
        const float* row = part + ((int64_t)s * n + t) * pg;
        if (i0 <= M) a0 += row[i0];
        if (i1 <= M) a1 += row[i1];
    }
    const float ss = M < 64 ? __shfl(a0, M) : __shfl(a1, M - 64);
    const float rstd = 1.0f / sqrtf(ss / (float)((int64_t)hc * d) + norm_eps);
    if (i0 < M) mixes[t * M + i0] = a0 * rstd;
    if (i1 < M) mixes[t * M + i1] = a1 * rstd;
}

int64_t ceil_div_g(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct GenericPlan {
    int64_t tiles;
    int cols_per_split;
    int nsplit;
    int pg;             // floats per partial row: (2+hc)hc dots + the sum of squares, padded to 4
    size_t part_bytes;
    size_t mixes_offset;  // scratch mixes after the partial rows (fused step)
    size_t total_bytes;
};

GenericPlan plan_generic(int64_t n, int hc, int64_t d) {
    GenericPlan p{};
    const int M = (2 + hc) * hc;
    const int64_t K = (int64_t)hc * d;
    p.tiles = ceil_div_g(n, kGTok);
    const int64_t ncols = ceil_div_g(K, kGCols);
    int64_t ns = ceil_div_g(512, p.tiles > 0 ? p.tiles : 1);   // about two workgroups per CU
    if (ns > ncols) ns = ncols;
    if (ns > kGMaxSplit) ns = kGMaxSplit;
    if (ns < 1) ns = 1;
    p.cols_per_split = (int)(ceil_div_g(ncols, ns) * kGCols);
    p.nsplit = (int)ceil_div_g(K, p.cols_per_split);
    p.pg = (M + 1 + 3) & ~3;
    p.part_bytes = (size_t)p.nsplit * (size_t)n * (size_t)p.pg * sizeof(float);
    p.mixes_offset = (p.part_bytes + 255) & ~size_t(255);
    p.total_bytes = p.mixes_offset + (size_t)n * (size_t)M * sizeof(float);
    return p;
}

template <bool kBf16>
void launch_partial(const GenericPlan& p, const void* x, const float* hc_fn, int64_t n, int hc, int64_t d,
                    float* part, hipStream_t stream) {
    const int M = (2 + hc) * hc;
    const dim3 grid((unsigned)(p.tiles * p.nsplit)), block(kGBlock);
    switch ((M + 15) / 16) {
        case 1: hipLaunchKernelGGL((mixes_partial_kernel<kBf16, 1>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                   p.cols_per_split, p.nsplit, part, p.pg); break;
        case 2: hipLaunchKernelGGL((mixes_partial_kernel<kBf16, 2>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                   p.cols_per_split, p.nsplit, part, p.pg); break;
        case 3: hipLaunchKernelGGL((mixes_partial_kernel<kBf16, 3>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                   p.cols_per_split, p.nsplit, part, p.pg); break;
        case 4: hipLaunchKernelGGL((mixes_partial_kernel<kBf16, 4>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                   p.cols_per_split, p.nsplit, part, p.pg); break;
        default: hipLaunchKernelGGL((mixes_partial_kernel<kBf16, 5>), grid, block, 0, stream, x, hc_fn, n, hc, d,
                                    p.cols_per_split, p.nsplit, part, p.pg); break;
    }
}

}  // namespace

size_t generic_workspace_bytes(int64_t n, int hc, int64_t d) { return plan_generic(n, hc, d).total_bytes; }

hipError_t launch_split_generic(const float* mixes, const float* scale, const float* base, int64_t n, int hc,
                                int iters, float eps, float* pre, float* post, float* comb, hipStream_t stream) {
    hipLaunchKernelGGL(split_generic_kernel, dim3((unsigned)ceil_div_g(n, kGBlock / 64)), dim3(kGBlock), 0, stream,
                       mixes, scale, base, n, hc, iters, eps, pre, post, comb);
    return hipGetLastError();
}

hipError_t launch_pre_generic(const void* x, bool bf16, const float* pre_mix, int64_t n, int hc, int64_t d, void* y,
                              hipStream_t stream) {
    const dim3 grid((unsigned)ceil_div_g(n * (d / 8), kGBlock));
    if (bf16)
        hipLaunchKernelGGL(pre_generic_kernel<true>, grid, dim3(kGBlock), 0, stream, x, pre_mix, n, hc, d, y);
    else
        hipLaunchKernelGGL(pre_generic_kernel<false>, grid, dim3(kGBlock), 0, stream, x, pre_mix, n, hc, d, y);
    return hipGetLastError();
}

hipError_t launch_post_generic(const void* f, const void* res, bool bf16, const float* post, const float* comb,
                               int64_t n, int hc, int64_t d, void* out, hipStream_t stream) {
    const dim3 grid((unsigned)ceil_div_g(n * (d / 8), kGBlock));
    if (bf16)
        hipLaunchKernelGGL(post_generic_kernel<true>, grid, dim3(kGBlock), 0, stream, f, res, post, comb, n, hc, d,
                           out);
    else
        hipLaunchKernelGGL(post_generic_kernel<false>, grid, dim3(kGBlock), 0, stream, f, res, post, comb, n, hc, d,
                           out);
    return hipGetLastError();
}

hipError_t launch_mixes_generic(const void* x, bool bf16, int64_t n, int hc, int64_t d, const float* hc_fn,
                                float norm_eps, float* mixes, void* workspace, hipStream_t stream) {
    const GenericPlan p = plan_generic(n, hc, d);
    float* part = static_cast<float*>(workspace);
    if (bf16)
        launch_partial<true>(p, x, hc_fn, n, hc, d, part, stream);
    else
        launch_partial<false>(p, x, hc_fn, n, hc, d, part, stream);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL(mixes_finalize_kernel, dim3((unsigned)ceil_div_g(n, kGBlock / 64)), dim3(kGBlock), 0, stream,
                       part, p.nsplit, p.pg, n, hc, d, norm_eps, mixes);
    return hipGetLastError();
}

hipError_t launch_fused_generic(const GenericRequest& r, hipStream_t stream) {
    const GenericPlan p = plan_generic(r.n, r.hc, r.d);
    const void* src = r.res;
    if (r.f_prev) {
        if (hipError_t e = launch_post_generic(r.f_prev, r.res, r.bf16, r.post_prev, r.comb_prev, r.n, r.hc, r.d,
                                               r.streams_out, stream);
            e != hipSuccess)
            return e;
        src = r.streams_out;
    }
    float* mixes = r.mixes ? r.mixes
                           : reinterpret_cast<float*>(static_cast<char*>(r.workspace) + p.mixes_offset);
    if (hipError_t e = launch_mixes_generic(src, r.bf16, r.n, r.hc, r.d, r.hc_fn, r.norm_eps, mixes, r.workspace,
                                            stream);
        e != hipSuccess)
        return e;
    if (hipError_t e = launch_split_generic(mixes, r.scale, r.base, r.n, r.hc, r.iters, r.eps, r.pre, r.post,
                                            r.comb, stream);
        e != hipSuccess)
        return e;
    if (r.y) return launch_pre_generic(src, r.bf16, r.pre_mix, r.n, r.hc, r.d, r.y, stream);
    return hipSuccess;
}

}  // namespace hc
