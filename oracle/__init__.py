"""CPU oracle for the hyper-connection residual mix -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library never imports, links or
calls it, and it imports nothing from the HIP library.

The arithmetic lives in ``hc_oracle.c`` (plain C, fp64 accumulation, one rounding
per materialised tensor). This module only marshals torch CPU tensors into it
and composes the steps into the sublayer order of ``Block.forward``.

Sources: atlas page "Block" (code section: ``Block.forward``, ``hc_mixes``,
``hc_pre``, ``hc_post``; parameter table), atlas page "Stream combination"
(summary, code section, released configuration), and the "DeepSeek-V4.1-Flash"
diagram (blocks "Mixing Coefficients", "First Sinkhorn Round", "Sinkhorn Round",
"Single-Pass mHC").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hc_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle_hc.so")

F32, BF16 = 0, 1

# Released configuration values ("Stream combination" page, configuration listing).
HC_MULT = 4
SINKHORN_ITERS = 20
HC_EPS = 1e-6
NORM_EPS = 1e-20

_lib = None


def build(sanitize: bool = False, src: str = _SRC, out: str | None = None,
          werror: bool = True) -> str:
    """Compile hc_oracle.c into liboracle_hc.so with gcc (no fast-math)."""
    if out is None:
        out = LIB_PATH if not sanitize else os.path.join(_HERE, "liboracle_hc_san.so")
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", out + ".tmp", "-lm"]
    if werror:
        cmd.insert(-5, "-Werror")
    if sanitize:
        # every finding is fatal (no recovery), so a sanitized run fails loudly
        cmd[1:1] = ["-fsanitize=address,undefined", "-fsanitize=float-cast-overflow",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("HC_ORACLE_LIB", LIB_PATH)  # the mutation test points this elsewhere
    if path == LIB_PATH and not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(path)
    P, I64, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.oracle_hc_mixes.argtypes = [P, I, I64, I, I64, P, D, P]
    lib.oracle_hc_split_sinkhorn.argtypes = [P, P, P, I64, I, I, D, P, P, P]
    lib.oracle_hc_pre.argtypes = [P, I, P, I64, I, I64, P]
    lib.oracle_hc_post.argtypes = [P, P, I, P, P, I64, I, I64, P]
    lib.oracle_round_bf16.argtypes = [D]
    lib.oracle_rmsnorm.argtypes = [P, I, I64, I64, P, D, P]
    lib.oracle_mxfp8.argtypes = [P, I, I64, I64, P, P]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    for name in ("oracle_hc_mixes", "oracle_hc_split_sinkhorn", "oracle_hc_pre", "oracle_hc_post"):
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"oracle supports fp32 and bf16 streams, got {t.dtype}")


def _cpu(t: torch.Tensor, dtype=None) -> torch.Tensor:
    t = t.detach().to("cpu")
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous()


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad argument (rc={rc})")


def round_bf16_bits(v: float) -> int:
    """Raw 16-bit word of the oracle's round-to-nearest-even bf16 of ``v``."""
    return int(_load().oracle_round_bf16(float(v)))


def hc_mixes(x: torch.Tensor, hc_fn: torch.Tensor, norm_eps: float = NORM_EPS) -> torch.Tensor:
    """x [..., hc, d] (fp32 or bf16), hc_fn [(2+hc)*hc, hc*d] fp32 -> mixes [..., (2+hc)*hc] fp32."""
    lib = _load()
    *lead, hc, d = x.shape
    n = int(torch.tensor(lead).prod()) if lead else 1
    xc = _cpu(x)
    w = _cpu(hc_fn, torch.float32)
    M = (2 + hc) * hc
    assert tuple(w.shape) == (M, hc * d), (tuple(w.shape), M, hc * d)
    out = torch.empty(*lead, M, dtype=torch.float32)
    _check(lib.oracle_hc_mixes(_ptr(xc), _dtype_code(xc), n, hc, d, _ptr(w), float(norm_eps),
                               _ptr(out)), "hc_mixes")
    return out


def hc_split_sinkhorn(mixes: torch.Tensor, hc_scale: torch.Tensor, hc_base: torch.Tensor,
                      hc_mult: int = HC_MULT, sinkhorn_iters: int = SINKHORN_ITERS,
                      eps: float = HC_EPS):
    """mixes [..., (2+hc)*hc] -> (pre [..., hc], post [..., hc], comb [..., hc, hc]), all fp32."""
    lib = _load()
    hc = hc_mult
    M = (2 + hc) * hc
    *lead, m = mixes.shape
    assert m == M, (m, M)
    n = int(torch.tensor(lead).prod()) if lead else 1
    mx = _cpu(mixes, torch.float32)
    s = _cpu(hc_scale, torch.float32)
    b = _cpu(hc_base, torch.float32)
    assert s.numel() == 3 and b.numel() == M
    pre = torch.empty(*lead, hc, dtype=torch.float32)
    post = torch.empty(*lead, hc, dtype=torch.float32)
    comb = torch.empty(*lead, hc, hc, dtype=torch.float32)
    _check(lib.oracle_hc_split_sinkhorn(_ptr(mx), _ptr(s), _ptr(b), n, hc, int(sinkhorn_iters),
                                        float(eps), _ptr(pre), _ptr(post), _ptr(comb)),
           "hc_split_sinkhorn")
    return pre, post, comb


def hc_pre(x: torch.Tensor, pre_mix: torch.Tensor) -> torch.Tensor:
    """x [..., hc, d], pre_mix [..., hc] fp32 -> y [..., d] in x's dtype."""
    lib = _load()
    *lead, hc, d = x.shape
    n = int(torch.tensor(lead).prod()) if lead else 1
    xc = _cpu(x)
    p = _cpu(pre_mix, torch.float32)
    y = torch.empty(*lead, d, dtype=xc.dtype)
    _check(lib.oracle_hc_pre(_ptr(xc), _dtype_code(xc), _ptr(p), n, hc, d, _ptr(y)), "hc_pre")
    return y


def hc_post(f: torch.Tensor, residual: torch.Tensor, post: torch.Tensor,
            comb: torch.Tensor) -> torch.Tensor:
    """f [..., d], residual [..., hc, d] (same dtype), post [..., hc], comb [..., hc, hc]
    -> new streams [..., hc, d] in f's dtype."""
    lib = _load()
    *lead, hc, d = residual.shape
    n = int(torch.tensor(lead).prod()) if lead else 1
    fc = _cpu(f)
    rc = _cpu(residual)
    if fc.dtype != rc.dtype:
        raise TypeError("oracle hc_post needs f and residual of one dtype")
    pc = _cpu(post, torch.float32)
    cc = _cpu(comb, torch.float32)
    out = torch.empty(*lead, hc, d, dtype=fc.dtype)
    _check(lib.oracle_hc_post(_ptr(fc), _ptr(rc), _dtype_code(fc), _ptr(pc), _ptr(cc), n, hc, d,
                              _ptr(out)), "hc_post")
    return out


def hc_mixes_split(x, hc_fn, hc_scale, hc_base, hc_mult=HC_MULT, sinkhorn_iters=SINKHORN_ITERS,
                   eps=HC_EPS, norm_eps=NORM_EPS):
    """The composite ``Block.hc_mixes``: projection, then split and Sinkhorn."""
    m = hc_mixes(x, hc_fn, norm_eps)
    pre, post, comb = hc_split_sinkhorn(m, hc_scale, hc_base, hc_mult, sinkhorn_iters, eps)
    return m, pre, post, comb


def fused_step(residual, hc_fn, hc_scale, hc_base, pre_mix, f_prev=None, post_prev=None,
               comb_prev=None, sinkhorn_iters=SINKHORN_ITERS, eps=HC_EPS, norm_eps=NORM_EPS):
    """One sublayer boundary in the order of ``Block.forward`` ("Single-Pass mHC").

    If ``f_prev`` is given, the previous sublayer's output is first written back
    into the streams (hc_post with post_prev / comb_prev); otherwise ``residual``
    is used as is. From the resulting streams the coefficients for THIS sublayer
    are computed (mixes, split, Sinkhorn), and the streams are collapsed with the
    collapse weights ``pre_mix`` handed over by the previous sublayer.
    Returns dict(streams, y, mixes, pre, post, comb).
    """
    hc = residual.shape[-2]
    streams = residual if f_prev is None else hc_post(f_prev, residual, post_prev, comb_prev)
    m, pre, post, comb = hc_mixes_split(streams, hc_fn, hc_scale, hc_base, hc, sinkhorn_iters,
                                        eps, norm_eps)
    y = hc_pre(streams, pre_mix)
    return dict(streams=streams, y=y, mixes=m, pre=pre, post=post, comb=comb)


def block(x, pre_mix, attn, ffn, f_attn, f_ffn, sinkhorn_iters=SINKHORN_ITERS, eps=HC_EPS,
          norm_eps=NORM_EPS):
    """The hyper-connection part of ``Block.forward`` with the sublayer bodies replaced
    by given outputs ``f_attn`` / ``f_ffn``.

    attn / ffn: (hc_fn, hc_scale, hc_base) of each sublayer.
    Attention collapses with ``pre_mix`` (handed over by the previous layer); the FFN
    collapses with the pre weights attention computed; the FFN's own pre weights are
    returned for the next layer.
    """
    hc = x.shape[-2]
    mA, preA, postA, combA = hc_mixes_split(x, *attn, hc, sinkhorn_iters, eps, norm_eps)
    yA = hc_pre(x, pre_mix)
    x1 = hc_post(f_attn, x, postA, combA)
    mF, preF, postF, combF = hc_mixes_split(x1, *ffn, hc, sinkhorn_iters, eps, norm_eps)
    yF = hc_pre(x1, preA)
    x2 = hc_post(f_ffn, x1, postF, combF)
    return dict(yA=yA, mixesA=mA, preA=preA, postA=postA, combA=combA, x1=x1,
                yF=yF, mixesF=mF, preF=preF, postF=postF, combF=combF, x2=x2)


def rmsnorm(x: torch.Tensor, gain: torch.Tensor, norm_eps: float = NORM_EPS) -> torch.Tensor:
    """RMSNorm of the collapsed input over its last (channel) axis, with a learned
    per-channel gain; result in the dtype of x. x: [..., d], gain: [d] fp32."""
    d = x.shape[-1]
    xc = _cpu(x)
    g = _cpu(gain, torch.float32)
    out = torch.empty_like(xc)
    n = xc.numel() // d
    _check(_load().oracle_rmsnorm(_ptr(xc), _dtype_code(xc), n, d, _ptr(g), norm_eps, _ptr(out)), "rmsnorm")
    return out


def mxfp8(x: torch.Tensor):
    """MXFP8 cast over the last axis (groups of 32 channels): returns (codes uint8
    [..., d] in E4M3, scales uint8 [..., d/32] in UE8M0)."""
    d = x.shape[-1]
    xc = _cpu(x)
    n = xc.numel() // d
    q = torch.empty(xc.shape, dtype=torch.uint8)
    sc = torch.empty(*xc.shape[:-1], d // 32, dtype=torch.uint8)
    _check(_load().oracle_mxfp8(_ptr(xc), _dtype_code(xc), n, d, _ptr(q), _ptr(sc)), "mxfp8")
    return q, sc


def param_shapes(hc: int, d: int):
    """Parameter shapes of one stream-weight instance ("Block" page parameter table):
    hc_fn [(2+hc)*hc, hc*d], hc_base [(2+hc)*hc], hc_scale [3]."""
    M = (2 + hc) * hc
    return dict(hc_fn=(M, hc * d), hc_base=(M,), hc_scale=(3,))


def comb_param_indices(hc: int):
    """Which entries of (hc_base, hc_scale) the comb matrix owns: hc*hc offsets at
    base[2hc : 2hc+hc^2] and the third scale ("Stream combination" page parameters)."""
    return list(range(2 * hc, 2 * hc + hc * hc)), [2]
