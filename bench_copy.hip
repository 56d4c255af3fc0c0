// bench_copy.hip -- the plain-copy reference of the benchmark (bench.py).
//
// A grid-stride copy of 16-byte elements: every lane moves one element per
// iteration, a wave 1 KB of consecutive addresses, the grid sweeps the buffer in
// address order. It is the ceiling the hyper-connection kernels' HBM rates are
// compared with, and the dispatch whose FETCH_SIZE / WRITE_SIZE counters calibrate
// the counter-based traffic figures (it moves exactly 2 x bytes).
//
// Built by __graft_entry__.build() into bench_copy.so; C ABI:
//   int bench_copy(const void* src, void* dst, int64_t bytes, int nontemporal,
//                  int workgroups, void* stream)
// src, dst: device buffers of `bytes` bytes (a multiple of 16, 16-byte aligned);
// nontemporal != 0 writes with non-temporal stores; returns 0, or -1 on a bad
// argument (nothing is launched), or the HIP error code of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

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
