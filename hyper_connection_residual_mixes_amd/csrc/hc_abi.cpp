// hc_abi.cpp -- the extern "C" entry points of libhc.so (declared in include/hc.h).
// Every argument is checked here, before any HIP call; then the launchers in
// hc_kernels.hip enqueue the work on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "hc.h"
#include "hc_internal.h"

namespace {

constexpr int kHC = 4;
// Rows (tokens) per call: every grid dimension the launchers derive from n stays
// far below 2^31 workgroups.
constexpr int64_t kMaxRows = 0x7fffffff;

struct Span {
    const void* p;
    size_t bytes;
};

bool overlaps(Span a, Span b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}
bool identical(Span a, Span b) { return a.p == b.p && a.bytes == b.bytes; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(int dtype) { return dtype == HC_BF16 ? 2 : 4; }

int64_t launch_items(int64_t n, int hc, int64_t d) {
    return hc == kHC ? hc::max_launch_items(n, d) : hc::generic_max_launch_items(n, hc, d);
}

// Shape rules shared by the stream entry points. Returns HC_OK or an error.
int check_shape(int64_t n, int hc, int64_t d, int dtype) {
    // d <= 2^20 keeps every per-wave byte offset of the kernels within 31 bits
    if (n < 0 || n > kMaxRows || d < 1 || d > (int64_t(1) << 20)) return HC_ERR_SHAPE;
    if (dtype != HC_F32 && dtype != HC_BF16) return HC_ERR_UNSUPPORTED;
    if (hc < 1 || hc > hc::kMaxHC || d % 8 != 0) return HC_ERR_UNSUPPORTED;
    // every byte offset must fit comfortably in 63 bits
    if (n > 0 && (uint64_t)d > (uint64_t(1) << 40) / (uint64_t)n) return HC_ERR_SHAPE;
    // every grid the launchers form must fit the launch limit
    if (n > 0 && launch_items(n, hc, d) > hc::kMaxLaunchItems) return HC_ERR_SHAPE;
    return HC_OK;
}

size_t mix_count(int hc) { return (size_t)(2 + hc) * (size_t)hc; }

// Workspace of the projection for (n, hc, d): the single-pass plan for four
// streams, the unfused plan otherwise.
size_t ws_bytes(int64_t n, int hc, int64_t d) {
    return hc == kHC ? hc::workspace_bytes(n, d) : hc::generic_workspace_bytes(n, hc, d);
}

int check_eps(float v) { return (std::isfinite(v) && v >= 0.f) ? HC_OK : HC_ERR_ARG; }

int hip_status(hipError_t e) { return e == hipSuccess ? HC_OK : HC_ERR_HIP; }

// No output may overlap an input or another output, except the listed exact aliases.
int check_aliases(const Span* outs, int n_out, const Span* ins, int n_in, const Span* allowed_pairs,
                  int n_allowed) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < n_in; ++j) {
            if (!overlaps(outs[i], ins[j])) continue;
            // only an exact in-place alias of a listed (output, input) pair is allowed
            bool ok = false;
            for (int k = 0; k + 1 < 2 * n_allowed; k += 2)
                if (identical(outs[i], ins[j]) && identical(outs[i], allowed_pairs[k]) &&
                    identical(ins[j], allowed_pairs[k + 1]))
                    ok = true;
            if (!ok) return HC_ERR_ALIAS;
        }
        for (int j = i + 1; j < n_out; ++j)
            if (overlaps(outs[i], outs[j])) return HC_ERR_ALIAS;
    }
    return HC_OK;
}

}  // namespace

extern "C" {

int hc_abi_version(void) { return HC_ABI_VERSION; }

const char* hc_status_string(int status) {
    switch (status) {
        case HC_OK: return "ok";
        case HC_ERR_NULL: return "a required pointer is NULL";
        case HC_ERR_SHAPE: return "invalid shape (n < 0, d < 1 or too large)";
        case HC_ERR_UNSUPPORTED: return "unsupported configuration (hc must be 1..8, d a multiple of 8, dtype fp32 or bf16)";
        case HC_ERR_ALIGN: return "misaligned pointer (16 bytes required)";
        case HC_ERR_ARG: return "invalid argument (sinkhorn_iters < 1, or eps/norm_eps negative or not finite)";
        case HC_ERR_ALIAS: return "an output overlaps an input or another output";
        case HC_ERR_WORKSPACE: return "workspace missing or too small";
        case HC_ERR_HIP: return "the HIP runtime reported an error";
        case HC_ERR_SCRATCH:
            return "the call needs more scratch than the no-allocation entry point's static buffer holds";
        default: return "unknown status";
    }
}

size_t hc_workspace_size(int64_t n, int hc, int64_t d) {
    if (n <= 0 || check_shape(n, hc, d, HC_F32) != HC_OK) return 0;
    return ws_bytes(n, hc, d);
}

int hc_split_sinkhorn(const float* mixes, const float* hc_scale, const float* hc_base, int64_t n, int hc,
                      int sinkhorn_iters, float eps, float* pre, float* post, float* comb, void* stream) {
    if (n < 0 || n > kMaxRows) return HC_ERR_SHAPE;
    if (hc < 1 || hc > hc::kMaxHC) return HC_ERR_UNSUPPORTED;
    // a lane per token (four streams) or a wave per token (other counts)
    if (hc != kHC && n > hc::kMaxLaunchItems / 64) return HC_ERR_SHAPE;
    if (sinkhorn_iters < 1 || check_eps(eps) != HC_OK) return HC_ERR_ARG;
    if (n == 0) return HC_OK;
    if (!mixes || !hc_scale || !hc_base || !pre || !post || !comb) return HC_ERR_NULL;
    if (!aligned(mixes, 16) || !aligned(pre, 16) || !aligned(post, 16) || !aligned(comb, 16) ||
        !aligned(hc_scale, 4) || !aligned(hc_base, 4))
        return HC_ERR_ALIGN;
    const size_t un = (size_t)n, uh = (size_t)hc, M = mix_count(hc);
    const Span outs[] = {{pre, un * uh * 4}, {post, un * uh * 4}, {comb, un * uh * uh * 4}};
    const Span ins[] = {{mixes, un * M * 4}, {hc_scale, 12}, {hc_base, M * 4}};
    if (int rc = check_aliases(outs, 3, ins, 3, nullptr, 0)) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (hc != kHC)
        return hip_status(hc::launch_split_generic(mixes, hc_scale, hc_base, n, hc, sinkhorn_iters, eps, pre, post,
                                                   comb, s));
    return hip_status(hc::launch_split(mixes, hc_scale, hc_base, n, sinkhorn_iters, eps, pre, post, comb, s));
}

int hc_pre(const void* x, int dtype, const float* pre_mix, int64_t n, int hc, int64_t d, void* y,
           void* stream) {
    if (int rc = check_shape(n, hc, d, dtype)) return rc;
    if (n == 0) return HC_OK;
    if (!x || !pre_mix || !y) return HC_ERR_NULL;
    if (!aligned(x, 16) || !aligned(pre_mix, 16) || !aligned(y, 16)) return HC_ERR_ALIGN;
    const size_t es = elem_size(dtype), un = (size_t)n, ud = (size_t)d;
    const size_t uh = (size_t)hc;
    const Span outs[] = {{y, un * ud * es}};
    const Span ins[] = {{x, un * uh * ud * es}, {pre_mix, un * uh * 4}};
    if (int rc = check_aliases(outs, 1, ins, 2, nullptr, 0)) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (hc != kHC) return hip_status(hc::launch_pre_generic(x, dtype == HC_BF16, pre_mix, n, hc, d, y, s));
    return hip_status(hc::launch_pre(x, dtype == HC_BF16, pre_mix, n, d, y, s));
}

int hc_rmsnorm_mxfp8(const void* x, int dtype, const float* gain, int64_t n, int64_t d, float norm_eps,
                     void* y_norm, uint8_t* q, uint8_t* scale, void* stream) {
    if (n < 0 || d < 8 || d > (int64_t(1) << 20)) return HC_ERR_SHAPE;
    if (n > 0 && (uint64_t)d > (uint64_t(1) << 40) / (uint64_t)n) return HC_ERR_SHAPE;
    if (n > kMaxRows) return HC_ERR_SHAPE;                       // the documented row bound
    if (dtype != HC_F32 && dtype != HC_BF16) return HC_ERR_UNSUPPORTED;
    if (d % 8 != 0) return HC_ERR_UNSUPPORTED;
    if (check_eps(norm_eps) != HC_OK) return HC_ERR_ARG;
    if ((q == nullptr) != (scale == nullptr)) return HC_ERR_NULL;  // codes and scales come together
    if (q && d % 32 != 0) return HC_ERR_UNSUPPORTED;
    if (!y_norm && !q) return HC_ERR_ARG;                          // nothing to produce
    if (n == 0) return HC_OK;
    if (!x || !gain) return HC_ERR_NULL;
    if (!aligned(x, 16) || !aligned(gain, 16) || (y_norm && !aligned(y_norm, 16)) || (q && !aligned(q, 8)))
        return HC_ERR_ALIGN;
    const size_t es = elem_size(dtype), un = (size_t)n, ud = (size_t)d;
    const Span x_span{x, un * ud * es};
    const Span outs[] = {{y_norm, un * ud * es}, {q, q ? un * ud : 0}, {scale, scale ? un * (ud / 32) : 0}};
    const Span ins[] = {x_span, {gain, ud * 4}};
    const Span allowed[] = {{y_norm, un * ud * es}, x_span};         // in place: y_norm == x
    if (int rc = check_aliases(outs, 3, ins, 2, allowed, 1)) return rc;
    return hip_status(hc::launch_rmsnorm_mxfp8(x, dtype == HC_BF16, gain, n, d, norm_eps, y_norm, q, scale,
                                               static_cast<hipStream_t>(stream)));
}

int hc_post(const void* f, const void* residual, int dtype, const float* post, const float* comb, int64_t n,
            int hc, int64_t d, void* out, void* stream) {
    if (int rc = check_shape(n, hc, d, dtype)) return rc;
    if (n == 0) return HC_OK;
    if (!f || !residual || !post || !comb || !out) return HC_ERR_NULL;
    if (!aligned(f, 16) || !aligned(residual, 16) || !aligned(post, 16) || !aligned(comb, 16) ||
        !aligned(out, 16))
        return HC_ERR_ALIGN;
    const size_t es = elem_size(dtype), un = (size_t)n, ud = (size_t)d;
    const size_t uh = (size_t)hc;
    const Span res_span{residual, un * uh * ud * es};
    const Span outs[] = {{out, un * uh * ud * es}};
    const Span ins[] = {{f, un * ud * es}, res_span, {post, un * uh * 4}, {comb, un * uh * uh * 4}};
    const Span allowed[] = {outs[0], res_span};
    if (int rc = check_aliases(outs, 1, ins, 4, allowed, 1)) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (hc != kHC)
        return hip_status(hc::launch_post_generic(f, residual, dtype == HC_BF16, post, comb, n, hc, d, out, s,
                                                  outs[0].bytes >= (size_t)hc::kStreamOutBytes));
    return hip_status(hc::launch_post(f, residual, dtype == HC_BF16, post, comb, n, d, out, s));
}

int hc_mixes(const void* x, int dtype, int64_t n, int hc, int64_t d, const float* hc_fn, float norm_eps,
             float* mixes, void* workspace, size_t workspace_bytes, void* stream) {
    if (int rc = check_shape(n, hc, d, dtype)) return rc;
    if (check_eps(norm_eps) != HC_OK) return HC_ERR_ARG;
    if (n == 0) return HC_OK;
    if (!x || !hc_fn || !mixes) return HC_ERR_NULL;
    if (!aligned(x, 16) || !aligned(hc_fn, 16) || !aligned(mixes, 16)) return HC_ERR_ALIGN;
    const size_t ws_need = ws_bytes(n, hc, d);
    if (!workspace || workspace_bytes < ws_need) return HC_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return HC_ERR_ALIGN;
    const size_t es = elem_size(dtype), un = (size_t)n, ud = (size_t)d, uh = (size_t)hc, M = mix_count(hc);
    const Span outs[] = {{mixes, un * M * 4}, {workspace, ws_need}};
    const Span ins[] = {{x, un * uh * ud * es}, {hc_fn, M * uh * ud * 4}};
    if (int rc = check_aliases(outs, 2, ins, 2, nullptr, 0)) return rc;
    if (hc != kHC)
        return hip_status(hc::launch_mixes_generic(x, dtype == HC_BF16, n, hc, d, hc_fn, norm_eps, mixes, workspace,
                                                   static_cast<hipStream_t>(stream)));
    hc::PassRequest r{};
    r.res = x;
    r.hc_fn = hc_fn;
    r.mixes = mixes;
    r.workspace = workspace;
    r.n = n;
    r.d = d;
    r.bf16 = dtype == HC_BF16;
    r.split = false;
    r.norm_eps = norm_eps;
    r.iters = 1;
    return hip_status(hc::launch_pass_and_finalize(r, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// hc_fused_step and hc_fused_step_noalloc. With noalloc the workspace arguments
// are ignored: the scratch is the library's static device array, looked up (the
// first HIP call) only after every argument has been validated.
int fused_step(const void* residual, const void* f_prev, const float* post_prev, const float* comb_prev,
               const float* pre_mix, const float* hc_fn, const float* hc_scale, const float* hc_base, int64_t n,
               int hc, int64_t d, int dtype, float norm_eps, int sinkhorn_iters, float eps, void* streams_out,
               void* y, float* pre, float* post, float* comb, float* mixes, void* workspace,
               size_t workspace_bytes, void* stream, bool noalloc) {
    if (int rc = check_shape(n, hc, d, dtype)) return rc;
    if (check_eps(norm_eps) != HC_OK || check_eps(eps) != HC_OK || sinkhorn_iters < 1) return HC_ERR_ARG;
    if (n == 0) return HC_OK;
    if (!residual || !hc_fn || !hc_scale || !hc_base || !pre || !post || !comb) return HC_ERR_NULL;
    const bool expand = f_prev != nullptr;
    if (expand && (!post_prev || !comb_prev || !streams_out)) return HC_ERR_NULL;
    if (y && !pre_mix) return HC_ERR_NULL;
    const size_t ws_need = ws_bytes(n, hc, d);
    if (noalloc) {
        if (ws_need > (size_t)HC_NOALLOC_SCRATCH_BYTES) return HC_ERR_SCRATCH;
        workspace = nullptr;   // the static scratch: no caller memory to check
        workspace_bytes = 0;
    } else if (!workspace || workspace_bytes < ws_need) {
        return HC_ERR_WORKSPACE;
    }
    const void* a16[] = {residual, hc_fn, pre, post, comb, workspace};
    for (const void* p : a16)
        if (p && !aligned(p, 16)) return HC_ERR_ALIGN;
    const void* o16[] = {f_prev, post_prev, comb_prev, pre_mix, streams_out, y, mixes};
    for (const void* p : o16)
        if (p && !aligned(p, 16)) return HC_ERR_ALIGN;
    if (!aligned(hc_scale, 4) || !aligned(hc_base, 4)) return HC_ERR_ALIGN;

    const size_t es = elem_size(dtype), un = (size_t)n, ud = (size_t)d, uh = (size_t)hc, M = mix_count(hc);
    const Span res_span{residual, un * uh * ud * es};
    const Span so_span{expand ? streams_out : nullptr, un * uh * ud * es};
    const Span outs[] = {so_span,
                         {y, un * ud * es},
                         {pre, un * uh * 4},
                         {post, un * uh * 4},
                         {comb, un * uh * uh * 4},
                         {mixes, un * M * 4},
                         {workspace, workspace ? ws_need : 0}};
    const Span ins[] = {res_span,
                        {f_prev, un * ud * es},
                        {expand ? post_prev : nullptr, un * uh * 4},
                        {expand ? comb_prev : nullptr, un * uh * uh * 4},
                        {y ? pre_mix : nullptr, un * uh * 4},
                        {hc_fn, M * uh * ud * 4},
                        {hc_scale, 12},
                        {hc_base, M * 4}};
    const Span allowed[] = {so_span, res_span};
    if (int rc = check_aliases(outs, 7, ins, 8, allowed, 1)) return rc;
    if (noalloc) {
        if (hc::noalloc_scratch(static_cast<hipStream_t>(stream), &workspace) != hipSuccess) return HC_ERR_HIP;
    }

    if (hc != kHC) {
        hc::GenericRequest g{};
        g.res = residual;
        g.f_prev = f_prev;
        g.post_prev = post_prev;
        g.comb_prev = comb_prev;
        g.pre_mix = pre_mix;
        g.hc_fn = hc_fn;
        g.scale = hc_scale;
        g.base = hc_base;
        g.streams_out = expand ? streams_out : nullptr;
        g.y = y;
        g.mixes = mixes;
        g.pre = pre;
        g.post = post;
        g.comb = comb;
        g.workspace = workspace;
        g.n = n;
        g.hc = hc;
        g.d = d;
        g.bf16 = dtype == HC_BF16;
        g.norm_eps = norm_eps;
        g.iters = sinkhorn_iters;
        g.eps = eps;
        return hip_status(hc::launch_fused_generic(g, static_cast<hipStream_t>(stream)));
    }

    hc::PassRequest r{};
    r.res = residual;
    r.f_prev = f_prev;
    r.post_prev = post_prev;
    r.comb_prev = comb_prev;
    r.pre_mix = pre_mix;
    r.hc_fn = hc_fn;
    r.scale = hc_scale;
    r.base = hc_base;
    r.streams_out = expand ? streams_out : nullptr;
    r.y = y;
    r.mixes = mixes;
    r.pre = pre;
    r.post = post;
    r.comb = comb;
    r.workspace = workspace;
    r.n = n;
    r.d = d;
    r.bf16 = dtype == HC_BF16;
    r.split = true;
    r.norm_eps = norm_eps;
    r.iters = sinkhorn_iters;
    r.eps = eps;
    return hip_status(hc::launch_pass_and_finalize(r, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int hc_fused_step(const void* residual, const void* f_prev, const float* post_prev, const float* comb_prev,
                  const float* pre_mix, const float* hc_fn, const float* hc_scale, const float* hc_base,
                  int64_t n, int hc, int64_t d, int dtype, float norm_eps, int sinkhorn_iters, float eps,
                  void* streams_out, void* y, float* pre, float* post, float* comb, float* mixes,
                  void* workspace, size_t workspace_bytes, void* stream) {
    return fused_step(residual, f_prev, post_prev, comb_prev, pre_mix, hc_fn, hc_scale, hc_base, n, hc, d, dtype,
                      norm_eps, sinkhorn_iters, eps, streams_out, y, pre, post, comb, mixes, workspace,
                      workspace_bytes, stream, false);
}

int hc_fused_step_noalloc(const void* residual, const void* f_prev, const float* post_prev,
                          const float* comb_prev, const float* pre_mix, const float* hc_fn,
                          const float* hc_scale, const float* hc_base, int64_t n, int hc, int64_t d,
                          int dtype, float norm_eps, int sinkhorn_iters, float eps, void* streams_out,
                          void* y, float* pre, float* post, float* comb, float* mixes, void* stream) {
    return fused_step(residual, f_prev, post_prev, comb_prev, pre_mix, hc_fn, hc_scale, hc_base, n, hc, d, dtype,
                      norm_eps, sinkhorn_iters, eps, streams_out, y, pre, post, comb, mixes, nullptr, 0, stream,
                      true);
}

}  // extern "C"
