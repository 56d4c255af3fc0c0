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
// bench_mfma_bf16: back-to-back v_mfma_f32_16x16x32_bf16 (the instruction the
// projections use), eight independent accumulators per wave, no memory traffic
// inside the loop: the rate the matrix cores sustain for that instruction.
//
// Built by __graft_entry__.build() into bench_ceilings.so; C ABI:
//   int bench_copy(const void* src, void* dst, int64_t bytes, int nontemporal,
//                  int workgroups, void* stream)
//     src, dst: device buffers of `bytes` bytes (a multiple of 16, 16-byte
//     aligned); nontemporal != 0 writes with non-temporal stores.
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

extern "C" int bench_copy(const void* src, void* dst, int64_t bytes, int nontemporal, int workgroups, void* stream) {
    if (!src || !dst || bytes <= 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > (1 << 20)) return -1;
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0) return -1;
    const int64_t count = bytes / 16;
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
