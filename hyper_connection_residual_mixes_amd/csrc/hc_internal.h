// hc_internal.h -- launchers behind the C ABI (not part of the public interface).
// Callers have validated every argument; these functions only enqueue kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hc {

// How one sweep over n tokens x d channels is cut into workgroups: `tiles`
// tiles of 64 (or 128) tokens times `nsplit` channel slices of `chunks_per_split`
// 32-channel steps. Each (slice, token) writes one 32-float partial row.
struct PassPlan {
    bool wide;               // bf16: 128-token groups (bf16_sweep2_kernel)
    int64_t tiles;
    int nchunks;
    int chunks_per_split;
    int nsplit;
    size_t workspace_bytes;  // per-slice partial rows
};
PassPlan plan_pass(int64_t n, int64_t d, bool bf16);
// Workspace that covers the plans of both stream dtypes.
size_t workspace_bytes(int64_t n, int64_t d);
// Work-items of the largest grid any four-stream launcher forms for (n, d); a
// launch takes at most kMaxLaunchItems per dimension.
int64_t max_launch_items(int64_t n, int64_t d);
constexpr int64_t kMaxLaunchItems = (int64_t(1) << 32) - 1;

struct PassRequest {
    const void* res;         // streams entering the boundary [n][4][d]
    const void* f_prev;      // previous sublayer output [n][d], or null (no expand)
    const float* post_prev;  // [n][4]
    const float* comb_prev;  // [n][4][4]
    const float* pre_mix;    // [n][4] collapse weights (used when y != null)
    const float* hc_fn;      // [24][4d]
    const float* scale;      // [3]
    const float* base;       // [24]
    void* streams_out;       // [n][4][d] when f_prev != null
    void* y;                 // [n][d] or null
    float* mixes;            // [n][24] or null
    float* pre;              // [n][4]   (split only)
    float* post;             // [n][4]   (split only)
    float* comb;             // [n][4][4] (split only)
    void* workspace;         // >= plan_pass(n, d).workspace_bytes
    int64_t n;
    int64_t d;
    bool bf16;
    bool split;              // run split + Sinkhorn after the projection
    float norm_eps;
    int iters;
    float eps;
};

hipError_t launch_split(const float* mixes, const float* scale, const float* base, int64_t n, int iters,
                        float eps, float* pre, float* post, float* comb, hipStream_t stream);
hipError_t launch_pre(const void* x, bool bf16, const float* pre_mix, int64_t n, int64_t d, void* y,
                      hipStream_t stream);
hipError_t launch_post(const void* f, const void* res, bool bf16, const float* post, const float* comb,
                       int64_t n, int64_t d, void* out, hipStream_t stream);
hipError_t launch_pass_and_finalize(const PassRequest& r, hipStream_t stream);
hipError_t launch_rmsnorm_mxfp8(const void* x, bool bf16, const float* gain, int64_t n, int64_t d, float eps,
                                void* y_norm, uint8_t* q, uint8_t* scale, hipStream_t stream);

// ------------------------------------------- stream counts other than four
// Unfused kernels for 1 <= hc <= kMaxHC (hc_generic.hip); four streams use the
// single-pass kernels above.
constexpr int kMaxHC = 8;

// Expand outputs of at least this many bytes (hc_post) are streamed to HBM with
// non-temporal stores: a quarter of the 256 MB last-level cache and well beyond
// the L2s, where keeping them cached would only defer their write-back into the
// next kernel's reads.
constexpr int64_t kStreamOutBytes = int64_t(64) << 20;

struct GenericRequest {
    const void* res;         // [n][hc][d]
    const void* f_prev;      // [n][d] or null (no expand)
    const float* post_prev;  // [n][hc]
    const float* comb_prev;  // [n][hc][hc]
    const float* pre_mix;    // [n][hc] (used when y != null)
    const float* hc_fn;      // [(2+hc)hc][hc d]
    const float* scale;      // [3]
    const float* base;       // [(2+hc)hc]
    void* streams_out;       // [n][hc][d] when f_prev != null (may be res)
    void* y;                 // [n][d] or null
    float* mixes;            // [n][(2+hc)hc] or null (then kept in the workspace)
    float* pre;
    float* post;
    float* comb;
    void* workspace;         // >= generic_workspace_bytes(n, hc, d)
    int64_t n;
    int hc;
    int64_t d;
    bool bf16;
    float norm_eps;
    int iters;
    float eps;
};

size_t generic_workspace_bytes(int64_t n, int hc, int64_t d);
int64_t generic_max_launch_items(int64_t n, int hc, int64_t d);

// Device address of the static no-allocation scratch (HC_NOALLOC_SCRATCH_BYTES)
// on the device of `stream`; looked up once per device (hc_noalloc.hip).
hipError_t noalloc_scratch(hipStream_t stream, void** out);
hipError_t launch_split_generic(const float* mixes, const float* scale, const float* base, int64_t n, int hc,
                                int iters, float eps, float* pre, float* post, float* comb, hipStream_t stream);
hipError_t launch_pre_generic(const void* x, bool bf16, const float* pre_mix, int64_t n, int hc, int64_t d, void* y,
                              hipStream_t stream);
hipError_t launch_post_generic(const void* f, const void* res, bool bf16, const float* post, const float* comb,
                               int64_t n, int hc, int64_t d, void* out, hipStream_t stream,
                               bool stream_out = false);
hipError_t launch_mixes_generic(const void* x, bool bf16, int64_t n, int hc, int64_t d, const float* hc_fn,
                                float norm_eps, float* mixes, void* workspace, hipStream_t stream);
hipError_t launch_fused_generic(const GenericRequest& r, hipStream_t stream);

}  // namespace hc
