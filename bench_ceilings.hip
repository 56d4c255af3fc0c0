// bench_ceilings.hip -- the measured ceilings the benchmark (bench.py) reports
// next to the published peaks.
//
// bench_copy: a grid-stride copy of 16-byte elements: every lane moves one
// element per iteration, a wave 1 KB of consecutive addresses, the grid sweeps
// the buffer in address order. It is the ceiling the hyper-connection kernels'
// HBM rates are compared with, and the dispatch whose FETCH_SIZE / WRITE_SIZE
// counters calibrate the counter-based traffic figures (it moves exactly
// 2 x bytes).
//
// bench_stream_mix: plain streaming with a given mix of read and written planes,
// laid out like the streams: `rows` rows (tokens), each holding its `nread`
// planes of `row_bytes` back to back (x[row][plane][channel]), and the outputs
// likewise. Element i (16 bytes) of every read plane of a row is combined and
// written to element i of every written plane of that row, grid-stride in address
// order. With 4 read / 1 written, 5 / 5 and 5 / 4 planes it is the ceiling of the
// attention boundary's, the FFN boundary's and the expand's flows without their
// arithmetic or their token-tiled walk.
//
// bench_empty: a kernel that does nothing, for the launch floor of a chain of
// dependent launches (the decode block replayed from a graph).
//
// bench_mfma_bf16: back-to-back v_mfma_f32_16x16x32_bf16 (the instruction the
// projections use), eight independent accumulators per wave, no memory traffic
// inside the loop: the rate the matrix cores sustain for that instruction. The
// file is built with the MFMA results in ordinary VGPRs (the build passes
// -amdgpu-mfma-vgpr-form): in the accumulation-register form the compiler
// rotates the eight accumulators through moves between the MFMAs of every
// iteration, which waits on each result and halves the measured rate.
//
// Built by __graft_entry__.build() into bench_ceilings.so; C ABI:
//   int bench_copy(const void* src, void* dst, int64_t bytes, int nontemporal,
//                  int workgroups, void* stream)
//     (for both copy and mix kernels, workgroups = 0 means one 16-byte element
//     per lane: a grid that covers the data once)
//     src, dst: device buffers of `bytes` bytes (a multiple of 16, 16-byte
//     aligned); nontemporal != 0 writes with non-temporal stores.
//   int bench_stream_mix(const void* src, void* dst, int64_t rows, int64_t row_bytes,
//                        int nread, int nwrite, int nontemporal, int workgroups,
//                        void* stream)
//     src: rows x nread x row_bytes, dst: rows x max(nwrite, 1) x row_bytes
//     (16-byte aligned, row_bytes a multiple of 16); 1 <= nread <= 5,
//     0 <= nwrite <= 5; with nwrite = 0 nothing is written (the loads are kept by
//     a comparison that never holds for the data the benchmark writes: all bytes 1).
//   int bench_empty(int workgroups, int threads, void* stream)
//     1 <= workgroups <= 2^20, 64 <= threads <= 1024 (a multiple of 64).
//   int bench_mfma_bf16(float* out, int64_t out_bytes, int workgroups, int iters,
//                       void* stream)
//     out: device buffer of at least workgroups * 256 floats (one sum per lane,
//     so the products are used); each workgroup of 4 waves issues
//     4 * iters * 8 MFMAs of 16 x 16 x 32 (16384 flops each).
// Both return 0, or -1 on a bad argument (nothing is launched), or the HIP
// error code of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

template <bool kNT>
__global__ __launch_bounds__(256) void copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                   int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
        const u32x4_t v = src[i];
        if constexpr (kNT) __builtin_nontemporal_store(v, dst + i);
        else dst[i] = v;
    }
}

template <int NR, int NW, bool kNT>
__global__ __launch_bounds__(256) void mix_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                  int64_t rows, int64_t row_elems) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x, count = rows * row_elems;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < count; k += stride) {
        const int64_t row = k / row_elems, i = k - row * row_elems;
        u32x4_t v[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) v[r] = src[(row * NR + r) * row_elems + i];
        u32x4_t acc = v[0];
#pragma unroll
        for (int r = 1; r < NR; ++r) acc += v[r];
        if constexpr (NW == 0) {
            if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) dst[k] = acc;   // never for all-ones bytes
        } else {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const u32x4_t o = acc + (unsigned)w;
                u32x4_t* q = dst + (row * NW + w) * row_elems + i;
                if constexpr (kNT) __builtin_nontemporal_store(o, q);
                else *q = o;
            }
        }
    }
}

template <int NR, int NW>
void launch_mix(const u32x4_t* src, u32x4_t* dst, int64_t rows, int64_t row_elems, bool nt, int wgs,
                hipStream_t s) {
    if (nt) hipLaunchKernelGGL((mix_kernel<NR, NW, true>), dim3(wgs), dim3(256), 0, s, src, dst, rows, row_elems);
    else hipLaunchKernelGGL((mix_kernel<NR, NW, false>), dim3(wgs), dim3(256), 0, s, src, dst, rows, row_elems);
}

template <int NR>
int launch_mix_r(const u32x4_t* src, u32x4_t* dst, int64_t rows, int64_t row_elems, int nw, bool nt, int wgs,
                 hipStream_t s) {
    switch (nw) {
        case 0: launch_mix<NR, 0>(src, dst, rows, row_elems, nt, wgs, s); break;
        case 1: launch_mix<NR, 1>(src, dst, rows, row_elems, nt, wgs, s); break;
        case 2: launch_mix<NR, 2>(src, dst, rows, row_elems, nt, wgs, s); break;
        case 3: launch_mix<NR, 3>(src, dst, rows, row_elems, nt, wgs, s); break;
        case 4: launch_mix<NR, 4>(src, dst, rows, row_elems, nt, wgs, s); break;
        case 5: launch_mix<NR, 5>(src, dst, rows, row_elems, nt, wgs, s); break;
        default: return -1;
    }
    return (int)hipGetLastError();
}

__global__ __launch_bounds__(1024) void empty_kernel() {}

__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ out, int iters) {
    bf16x8_t a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(threadIdx.x + i));
        b[i] = (__bf16)(0.002f * (float)i);
    }
    floatx4_t acc[8];
    for (int i = 0; i < 8; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.f;
    for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// workgroups == 0: one element per lane (a grid that covers the data once,
// dispatched in address order).
static int grid_for(int64_t count, int workgroups) {
    if (workgroups != 0) return workgroups;
    const int64_t g = (count + 255) / 256;
    return g > (1 << 20) ? -1 : (int)g;
}

extern "C" int bench_copy(const void* src, void* dst, int64_t bytes, int nontemporal, int workgroups, void* stream) {
    if (!src || !dst || bytes <= 0 || bytes % 16 != 0 || workgroups < 0 || workgroups > (1 << 20)) return -1;
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return -1;
    const int64_t count = bytes / 16;
    workgroups = grid_for(count, workgroups);
    if (workgroups < 1) return -1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (nontemporal)
        hipLaunchKernelGGL(copy_kernel<true>, dim3(workgroups), dim3(256), 0, s,
                           static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), count);
    else
        hipLaunchKernelGGL(copy_kernel<false>, dim3(workgroups), dim3(256), 0, s,
                           static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), count);
    return (int)hipGetLastError();
}

extern "C" int bench_mfma_bf16(float* out, int64_t out_bytes, int workgroups, int iters, void* stream) {
    if (!out || workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24)) return -1;
    if (out_bytes < (int64_t)workgroups * 256 * (int64_t)sizeof(float)) return -1;
    hipLaunchKernelGGL(mfma_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
    return (int)hipGetLastError();
}

extern "C" int bench_stream_mix(const void* src, void* dst, int64_t rows, int64_t row_bytes, int nread,
                                int nwrite, int nontemporal, int workgroups, void* stream) {
    if (!src || !dst || rows <= 0 || row_bytes <= 0 || row_bytes % 16 != 0 || nread < 1 || nread > 5 ||
        nwrite < 0 || nwrite > 5 || workgroups < 0 || workgroups > (1 << 20))
        return -1;
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return -1;
    const int64_t row_elems = row_bytes / 16;
    workgroups = grid_for(rows * row_elems, workgroups);
    if (workgroups < 1) return -1;
    const u32x4_t* s = static_cast<const u32x4_t*>(src);
    u32x4_t* d = static_cast<u32x4_t*>(dst);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const bool nt = nontemporal != 0;
    switch (nread) {
        case 1: return launch_mix_r<1>(s, d, rows, row_elems, nwrite, nt, workgroups, st);
        case 2: return launch_mix_r<2>(s, d, rows, row_elems, nwrite, nt, workgroups, st);
        case 3: return launch_mix_r<3>(s, d, rows, row_elems, nwrite, nt, workgroups, st);
        case 4: return launch_mix_r<4>(s, d, rows, row_elems, nwrite, nt, workgroups, st);
        default: return launch_mix_r<5>(s, d, rows, row_elems, nwrite, nt, workgroups, st);
    }
}

extern "C" int bench_empty(int workgroups, int threads, void* stream) {
    if (workgroups < 1 || workgroups > (1 << 20) || threads < 64 || threads > 1024 || threads % 64 != 0) return -1;
    hipLaunchKernelGGL(empty_kernel, dim3(workgroups), dim3(threads), 0, static_cast<hipStream_t>(stream));
    return (int)hipGetLastError();
}
