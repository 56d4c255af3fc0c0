"""Python binding of libhc.so, the gfx950 hyper-connection residual mix.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in ``include/hc.h``. PyTorch provides device memory (output and workspace
tensors) and the current HIP stream. There is no fallback: if the library is not
built, every call raises.

The functions carry the names of the C entry points. Shapes follow the pages'
``Block`` methods: streams [..., hc, d], sublayer input/output [..., d], mixes
[..., (2+hc)hc], pre/post [..., hc], comb [..., hc, hc]; hc = 4 in the released
configuration, 1..8 supported.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# HC_LIBRARY names another build of the same library (the host-sanitizer test uses it)
LIB_PATH = os.environ.get("HC_LIBRARY") or os.path.join(_PKG, "libhc.so")

HC_F32, HC_BF16 = 0, 1
HC_MULT, SINKHORN_ITERS, HC_EPS, NORM_EPS = 4, 20, 1e-6, 1e-20
MIX = (2 + HC_MULT) * HC_MULT

_lib = None


class HCError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text} (status {status})")
        self.status = status


def lib():
    """The loaded libhc.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run __graft_entry__.build() or hyper_connection_residual_mixes_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.hc_abi_version.restype = I
    L.hc_status_string.argtypes = [I]
    L.hc_status_string.restype = ctypes.c_char_p
    L.hc_workspace_size.argtypes = [I64, I, I64]
    L.hc_workspace_size.restype = SZ
    L.hc_mixes.argtypes = [P, I, I64, I, I64, P, F, P, P, SZ, P]
    L.hc_split_sinkhorn.argtypes = [P, P, P, I64, I, I, F, P, P, P, P]
    L.hc_pre.argtypes = [P, I, P, I64, I, I64, P, P]
    L.hc_post.argtypes = [P, P, I, P, P, I64, I, I64, P, P]
    L.hc_rmsnorm_mxfp8.argtypes = [P, I, P, I64, I64, F, P, P, P, P]
    L.hc_fused_step.argtypes = [P, P, P, P, P, P, P, P, I64, I, I64, I, F, I, F,
                                P, P, P, P, P, P, P, SZ, P]
    L.hc_fused_step_noalloc.argtypes = [P, P, P, P, P, P, P, P, I64, I, I64, I, F, I, F,
                                        P, P, P, P, P, P, P]
    for name in ("hc_mixes", "hc_split_sinkhorn", "hc_pre", "hc_post", "hc_fused_step", "hc_fused_step_noalloc",
                 "hc_rmsnorm_mxfp8"):
        getattr(L, name).restype = I
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().hc_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise HCError(fn, status, status_string(status))


def _ptr(t):
    # an int: ctypes converts it for the c_void_p argument
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device):
    """The current HIP stream of `device` (torch's), as an address."""
    if _raw_stream is not None and device.index is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HC_BF16
    if t.dtype == torch.float32:
        return HC_F32
    raise TypeError(f"stream dtype must be bfloat16 or float32, got {t.dtype}")


def _dev(t: torch.Tensor, what: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _size(t: torch.Tensor, count: int, what: str, device) -> torch.Tensor:
    """The library reads or writes exactly ``count`` elements behind each pointer: a
    tensor of another size, or on another device, is refused here rather than
    faulting the GPU."""
    if t.numel() != count:
        raise ValueError(f"{what} must hold {count} elements, got {t.numel()} (shape {tuple(t.shape)})")
    if t.get_device() != device.index:
        raise ValueError(f"{what} is on {t.device}, expected {device}")
    return t


def _streams_shape(x: torch.Tensor):
    if x.dim() < 2:
        raise ValueError("streams must have shape [..., hc, d]")
    *lead, hc, d = x.shape
    n = 1
    for s in lead:
        n *= s
    return lead, n, hc, d


def workspace_size(n: int, hc: int, d: int) -> int:
    return int(lib().hc_workspace_size(n, hc, d))


def _workspace(n, hc, d, device, workspace):
    """The caller's workspace (its size is checked by the library), or a new one."""
    if workspace is None:
        workspace = torch.empty(max(workspace_size(n, hc, d), 16), dtype=torch.uint8, device=device)
    _dev(workspace, "workspace")
    if workspace.device != device:
        raise ValueError(f"workspace is on {workspace.device}, expected {device}")
    return workspace, workspace.numel() * workspace.element_size()


def hc_mixes(x, hc_fn, norm_eps=NORM_EPS, out=None, workspace=None):
    """x [..., hc, d] -> mixes [..., (2+hc)hc] fp32 (projection scaled by the RMS statistic)."""
    _dev(x, "x")
    _dev(hc_fn, "hc_fn", torch.float32)
    lead, n, hc, d = _streams_shape(x)
    M = (2 + hc) * hc
    _size(hc_fn, M * hc * d, "hc_fn", x.device)
    if out is None:
        out = torch.empty(*lead, M, dtype=torch.float32, device=x.device)
    _size(_dev(out, "mixes", torch.float32), n * M, "mixes", x.device)
    ws, ws_bytes = _workspace(n, hc, d, x.device, workspace)
    _check("hc_mixes", lib().hc_mixes(_ptr(x), _dtype_code(x), n, hc, d, _ptr(hc_fn), float(norm_eps),
                                      _ptr(out), _ptr(ws), ws_bytes, _stream(x.device)))
    return out


def hc_split_sinkhorn(mixes, hc_scale, hc_base, hc_mult=HC_MULT, sinkhorn_iters=SINKHORN_ITERS,
                      eps=HC_EPS, out=None):
    """mixes [..., (2+hc)hc] -> (pre [..., hc], post [..., hc], comb [..., hc, hc]), fp32,
    hc = hc_mult."""
    _dev(mixes, "mixes", torch.float32)
    _dev(hc_scale, "hc_scale", torch.float32)
    _dev(hc_base, "hc_base", torch.float32)
    *lead, m = mixes.shape
    n = 1
    for s in lead:
        n *= s
    if out is None:
        out = (torch.empty(*lead, hc_mult, dtype=torch.float32, device=mixes.device),
               torch.empty(*lead, hc_mult, dtype=torch.float32, device=mixes.device),
               torch.empty(*lead, hc_mult, hc_mult, dtype=torch.float32, device=mixes.device))
    pre, post, comb = (_dev(t, nm, torch.float32) for t, nm in zip(out, ("pre", "post", "comb")))
    if m != (2 + hc_mult) * hc_mult:
        raise ValueError(f"mixes last dim must be {(2 + hc_mult) * hc_mult}, got {m}")
    dev = mixes.device
    _size(hc_scale, 3, "hc_scale", dev)
    _size(hc_base, m, "hc_base", dev)
    _size(pre, n * hc_mult, "pre", dev)
    _size(post, n * hc_mult, "post", dev)
    _size(comb, n * hc_mult * hc_mult, "comb", dev)
    _check("hc_split_sinkhorn", lib().hc_split_sinkhorn(
        _ptr(mixes), _ptr(hc_scale), _ptr(hc_base), n, hc_mult, int(sinkhorn_iters), float(eps),
        _ptr(pre), _ptr(post), _ptr(comb), _stream(mixes.device)))
    return pre, post, comb


def hc_pre(x, pre_mix, out=None):
    """Collapse: x [..., hc, d], pre_mix [..., hc] -> y [..., d] in x's dtype."""
    _dev(x, "x")
    _dev(pre_mix, "pre_mix", torch.float32)
    lead, n, hc, d = _streams_shape(x)
    _size(pre_mix, n * hc, "pre_mix", x.device)
    if out is None:
        out = torch.empty(*lead, d, dtype=x.dtype, device=x.device)
    _size(_dev(out, "y", x.dtype), n * d, "y", x.device)
    _check("hc_pre", lib().hc_pre(_ptr(x), _dtype_code(x), _ptr(pre_mix), n, hc, d, _ptr(out),
                                  _stream(x.device)))
    return out


def hc_post(f, residual, post, comb, out=None):
    """Expand and combine: new stream k = post[k] f + sum_j comb[j][k] residual[j]."""
    _dev(f, "f")
    _dev(residual, "residual", f.dtype)
    _dev(post, "post", torch.float32)
    _dev(comb, "comb", torch.float32)
    lead, n, hc, d = _streams_shape(residual)
    dev = residual.device
    _size(f, n * d, "f", dev)
    _size(post, n * hc, "post", dev)
    _size(comb, n * hc * hc, "comb", dev)
    if out is None:
        out = torch.empty_like(residual)
    _size(_dev(out, "out", f.dtype), n * hc * d, "out", dev)
    _check("hc_post", lib().hc_post(_ptr(f), _ptr(residual), _dtype_code(f), _ptr(post), _ptr(comb), n,
                                    hc, d, _ptr(out), _stream(f.device)))
    return out


def rmsnorm_mxfp8(x, gain, norm_eps=NORM_EPS, want_norm=True, want_cast=True, y_norm=None, q=None,
                  scale=None):
    """The sublayer RMSNorm (learned gain) of a collapsed input x [..., d] and its
    MXFP8 cast (groups of 32 channels). Returns dict(y_norm, q, scale): y_norm in
    x's dtype, q E4M3 codes uint8 [..., d], scale UE8M0 bytes uint8 [..., d/32];
    entries not requested are None."""
    _dev(x, "x")
    _dev(gain, "gain", torch.float32)
    d = x.shape[-1]
    n = x.numel() // d if d else 0
    _size(gain, d, "gain", x.device)
    if want_norm and y_norm is None:
        y_norm = torch.empty_like(x)
    if want_norm:
        _size(_dev(y_norm, "y_norm", x.dtype), n * d, "y_norm", x.device)
    if want_cast:
        if q is None:
            q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
        if scale is None:
            scale = torch.empty(*x.shape[:-1], d // 32, dtype=torch.uint8, device=x.device)
        _size(_dev(q, "q", torch.uint8), n * d, "q", x.device)
        _size(_dev(scale, "scale", torch.uint8), n * (d // 32), "scale", x.device)
    else:
        q = scale = None
    _check("hc_rmsnorm_mxfp8", lib().hc_rmsnorm_mxfp8(
        _ptr(x), _dtype_code(x), _ptr(gain), n, d, float(norm_eps), _ptr(y_norm) if want_norm else None,
        _ptr(q), _ptr(scale), _stream(x.device)))
    return dict(y_norm=y_norm if want_norm else None, q=q, scale=scale)


def hc_fused_step(residual, hc_fn, hc_scale, hc_base, pre_mix=None, f_prev=None, post_prev=None,
                  comb_prev=None, sinkhorn_iters=SINKHORN_ITERS, eps=HC_EPS, norm_eps=NORM_EPS,
                  streams_out=None, y=None, out=None, want_mixes=False, want_y=True, workspace=None):
    """One sublayer boundary: optional expand of the previous sublayer's output, then
    this sublayer's coefficients and the collapse with ``pre_mix``.

    Returns dict(streams, y, pre, post, comb, mixes) (streams is ``residual`` when
    ``f_prev`` is None; y / mixes are None when not requested; ``want_mixes`` may
    also be the output tensor itself)."""
    return _fused_step(residual, hc_fn, hc_scale, hc_base, pre_mix, f_prev, post_prev, comb_prev,
                       sinkhorn_iters, eps, norm_eps, streams_out, y, out, want_mixes, want_y, workspace,
                       noalloc=False)


def hc_fused_step_noalloc(residual, hc_fn, hc_scale, hc_base, pre_mix=None, f_prev=None, post_prev=None,
                          comb_prev=None, sinkhorn_iters=SINKHORN_ITERS, eps=HC_EPS, norm_eps=NORM_EPS,
                          streams_out=None, y=None, out=None, want_mixes=False, want_y=True):
    """``hc_fused_step`` on the library's static device scratch instead of a
    workspace (C entry point ``hc_fused_step_noalloc``). The library allocates
    nothing; with every output tensor passed in, neither does this call."""
    return _fused_step(residual, hc_fn, hc_scale, hc_base, pre_mix, f_prev, post_prev, comb_prev,
                       sinkhorn_iters, eps, norm_eps, streams_out, y, out, want_mixes, want_y, None,
                       noalloc=True)


def _fused_step(residual, hc_fn, hc_scale, hc_base, pre_mix, f_prev, post_prev, comb_prev, sinkhorn_iters,
                eps, norm_eps, streams_out, y, out, want_mixes, want_y, workspace, noalloc):
    _dev(residual, "residual")
    lead, n, hc, d = _streams_shape(residual)
    dev = residual.device
    expand = f_prev is not None
    M = (2 + hc) * hc
    _size(_dev(hc_fn, "hc_fn", torch.float32), M * hc * d, "hc_fn", dev)
    _size(_dev(hc_scale, "hc_scale", torch.float32), 3, "hc_scale", dev)
    _size(_dev(hc_base, "hc_base", torch.float32), M, "hc_base", dev)
    if expand:
        _size(_dev(f_prev, "f_prev", residual.dtype), n * d, "f_prev", dev)
        _size(_dev(post_prev, "post_prev", torch.float32), n * hc, "post_prev", dev)
        _size(_dev(comb_prev, "comb_prev", torch.float32), n * hc * hc, "comb_prev", dev)
        if streams_out is None:
            streams_out = torch.empty_like(residual)
        _size(_dev(streams_out, "streams_out", residual.dtype), n * hc * d, "streams_out", dev)
    if want_y:
        _size(_dev(pre_mix, "pre_mix", torch.float32), n * hc, "pre_mix", dev)
        if y is None:
            y = torch.empty(*lead, d, dtype=residual.dtype, device=dev)
        _size(_dev(y, "y", residual.dtype), n * d, "y", dev)
    else:
        y = None
    if out is None:
        out = (torch.empty(*lead, hc, dtype=torch.float32, device=dev),
               torch.empty(*lead, hc, dtype=torch.float32, device=dev),
               torch.empty(*lead, hc, hc, dtype=torch.float32, device=dev))
    pre, post, comb = out
    _size(_dev(pre, "pre", torch.float32), n * hc, "pre", dev)
    _size(_dev(post, "post", torch.float32), n * hc, "post", dev)
    _size(_dev(comb, "comb", torch.float32), n * hc * hc, "comb", dev)
    if isinstance(want_mixes, torch.Tensor):   # the caller's mixes tensor
        mixes = _size(_dev(want_mixes, "mixes", torch.float32), n * (2 + hc) * hc, "mixes", dev)
    elif want_mixes:
        mixes = torch.empty(*lead, (2 + hc) * hc, dtype=torch.float32, device=dev)
    else:
        mixes = None
    args = (_ptr(residual), _ptr(f_prev), _ptr(post_prev) if expand else None,
            _ptr(comb_prev) if expand else None, _ptr(pre_mix) if want_y else None,
            _ptr(hc_fn), _ptr(hc_scale), _ptr(hc_base), n, hc, d, _dtype_code(residual),
            float(norm_eps), int(sinkhorn_iters), float(eps), _ptr(streams_out) if expand else None,
            _ptr(y), _ptr(pre), _ptr(post), _ptr(comb), _ptr(mixes))
    if noalloc:
        _check("hc_fused_step_noalloc", lib().hc_fused_step_noalloc(*args, _stream(dev)))
    else:
        ws, ws_bytes = _workspace(n, hc, d, dev, workspace)
        _check("hc_fused_step", lib().hc_fused_step(*args, _ptr(ws), ws_bytes, _stream(dev)))
    return dict(streams=streams_out if expand else residual, y=y, pre=pre, post=post, comb=comb,
                mixes=mixes)


def block(x, pre_mix, attn, ffn, f_attn, f_ffn, sinkhorn_iters=SINKHORN_ITERS, eps=HC_EPS,
          norm_eps=NORM_EPS, x1_out=None, x2_out=None, workspace=None):
    """The hyper-connection part of one block (attention then FFN boundary) with the
    sublayer bodies replaced by the given outputs, as three launches-worth of work:
    fused(attention: coefficients + collapse), fused(expand attention output +
    FFN coefficients + collapse with attention's pre), expand(FFN output)."""
    a = hc_fused_step(x, *attn, pre_mix=pre_mix, sinkhorn_iters=sinkhorn_iters, eps=eps,
                      norm_eps=norm_eps, workspace=workspace)
    f = hc_fused_step(x, *ffn, pre_mix=a["pre"], f_prev=f_attn, post_prev=a["post"],
                      comb_prev=a["comb"], sinkhorn_iters=sinkhorn_iters, eps=eps, norm_eps=norm_eps,
                      streams_out=x1_out, workspace=workspace)
    x2 = hc_post(f_ffn, f["streams"], f["post"], f["comb"], out=x2_out)
    return dict(yA=a["y"], preA=a["pre"], postA=a["post"], combA=a["comb"], x1=f["streams"],
                yF=f["y"], preF=f["pre"], postF=f["post"], combF=f["comb"], x2=x2)
