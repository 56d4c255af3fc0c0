"""C-ABI checks that need no GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments before any HIP call.

Pointers passed here are fake addresses; every call below must fail validation, so
none of them reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

import torch

import hyper_connection_residual_mixes_amd as hc

# Fake addresses must never reach a device: these tests run only where no GPU exists.
pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-only validation tests (fake device pointers)")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hc.h")

OK, NULL, SHAPE, UNSUP, ALIGN, ARG, ALIAS, WS, HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8
P = ctypes.c_void_p
A = 0x10000000          # a 16-byte aligned fake address
B = 0x20000000
C = 0x30000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[a-z_ ]+[ *]+(hc_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("hc_mixes", "hc_split_sinkhorn", "hc_pre", "hc_post", "hc_fused_step", "hc_fused_step_noalloc",
                 "hc_rmsnorm_mxfp8", "hc_workspace_size", "hc_status_string", "hc_abi_version"):
        assert want in names


def test_library_exports_every_declared_symbol():
    L = hc.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_status_strings():
    L = hc.lib()
    assert L.hc_abi_version() == 1
    for s in range(-9, 1):
        assert hc.status_string(s) and hc.status_string(s) != "unknown status"
    assert hc.status_string(-99) == "unknown status"


def test_workspace_size_rule():
    # one 128-byte partial row per (channel slice, token); slices are whole 64-
    # (bf16) or 128-channel (fp32) steps, at most 128 of them
    assert hc.workspace_size(0, 4, 5120) == 0
    assert hc.workspace_size(16, 9, 5120) == 0
    assert hc.workspace_size(16, 0, 5120) == 0
    assert hc.workspace_size(16, 4, 12) == 0
    for n, d in ((16, 256), (64, 5120), (4096, 5120), (65536, 5120), (37, 264)):
        ws = hc.workspace_size(n, 4, d)
        assert ws > 0 and ws % (128 * n) == 0
        nsplit = ws // (128 * n)
        assert 1 <= nsplit <= min(128, -(-d // 64))
    # other stream counts: partial rows of (2+hc)hc dots + 1 sum of squares (padded
    # to 4 floats) per (slice, token), then n scratch mix rows
    for hc_, n, d in ((1, 16, 256), (2, 37, 264), (8, 64, 5120), (3, 4096, 5120)):
        M = (2 + hc_) * hc_
        pg = (M + 1 + 3) // 4 * 4
        ws = hc.workspace_size(n, hc_, d)
        assert ws >= n * pg * 4 + n * M * 4


def _split(mixes=A, scale=B, base=C, n=16, hc_=4, iters=20, eps=1e-6, pre=A + 4096, post=A + 8192,
           comb=A + 16384):
    return hc.lib().hc_split_sinkhorn(P(mixes), P(scale), P(base), n, hc_, iters, eps, P(pre), P(post),
                                      P(comb), None)


def test_split_validation():
    assert _split(n=0) == OK            # no-op touches nothing
    assert _split(n=-1) == SHAPE
    assert _split(hc_=9) == UNSUP
    assert _split(hc_=0) == UNSUP
    assert _split(iters=0) == ARG
    assert _split(eps=-1.0) == ARG
    assert _split(eps=float("nan")) == ARG
    assert _split(mixes=None) == NULL
    assert _split(mixes=A + 4) == ALIGN
    assert _split(pre=A) == ALIAS        # pre overlaps mixes
    assert _split(comb=A + 4096) == ALIAS  # comb overlaps pre


def _pre(x=A, dtype=1, pm=B, n=16, hc_=4, d=256, y=C):
    return hc.lib().hc_pre(P(x), dtype, P(pm), n, hc_, d, P(y), None)


def test_pre_validation():
    assert _pre(n=0) == OK
    assert _pre(d=0) == SHAPE
    assert _pre(d=260) == UNSUP
    assert _pre(d=(1 << 20) + 8) == SHAPE   # beyond the supported width
    assert _pre(dtype=2) == UNSUP
    assert _pre(hc_=9) == UNSUP
    assert _pre(hc_=0) == UNSUP
    assert _pre(x=None) == NULL
    assert _pre(y=C + 2) == ALIGN
    assert _pre(y=A + 1024) == ALIAS


def _post(f=A, res=B, dtype=1, post=C, comb=C + 4096, n=16, d=256, out=0x40000000):
    return hc.lib().hc_post(P(f), P(res), dtype, P(post), P(comb), n, 4, d, P(out), None)


def test_post_validation():
    assert _post(n=0) == OK
    assert _post(f=None) == NULL
    assert _post(comb=C + 8) == ALIGN
    assert _post(out=B + 16) == ALIAS    # partial overlap with residual
    assert _post(out=A) == ALIAS         # overlaps f


def _mixes(x=A, n=16, d=256, fn=B, norm_eps=1e-20, mixes=C, ws=0x40000000, ws_bytes=1 << 20):
    return hc.lib().hc_mixes(P(x), 1, n, 4, d, P(fn), norm_eps, P(mixes), P(ws), ws_bytes, None)


def test_mixes_validation():
    assert _mixes(n=0) == OK
    assert _mixes(norm_eps=-1.0) == ARG
    assert _mixes(ws=None) == WS
    assert _mixes(ws_bytes=hc.workspace_size(16, 4, 256) - 1) == WS
    assert _mixes(ws=0x40000008) == ALIGN
    assert _mixes(mixes=A + 256) == ALIAS
    assert _mixes(ws=C) == ALIAS


def _fused(res=A, f_prev=None, post_prev=None, comb_prev=None, pre_mix=0x50000000, fn=B, scale=C,
           base=C + 64, n=16, d=256, dtype=1, iters=20, so=None, y=0x60000000, pre=0x70000000,
           post=0x70001000, comb=0x70002000, mixes=None, ws=0x40000000, ws_bytes=1 << 20):
    return hc.lib().hc_fused_step(P(res), P(f_prev), P(post_prev), P(comb_prev), P(pre_mix), P(fn),
                                  P(scale), P(base), n, 4, d, dtype, 1e-20, iters, 1e-6, P(so), P(y),
                                  P(pre), P(post), P(comb), P(mixes), P(ws), ws_bytes, None)


def test_fused_validation():
    assert _fused(n=0) == OK
    assert _fused(iters=0) == ARG
    assert _fused(pre=None) == NULL
    assert _fused(f_prev=0x58000000) == NULL                       # expand needs post/comb/out
    assert _fused(pre_mix=None) == NULL                            # a collapse needs pre_mix
    assert _fused(ws_bytes=16) == WS
    assert _fused(scale=C + 2) == ALIGN
    assert _fused(y=A + 64) == ALIAS                               # y inside residual
    assert _fused(f_prev=0x58000000, post_prev=0x59000000, comb_prev=0x59001000,
                  so=A + 16) == ALIAS                              # partial overlap with residual
    assert _fused(mixes=0x70000080) == ALIAS                       # mixes inside pre


def _norm(x=A, dtype=1, gain=B, n=16, d=256, eps=1e-20, y=C, q=0x40000000, sc=0x50000000):
    return hc.lib().hc_rmsnorm_mxfp8(P(x), dtype, P(gain), n, d, eps, P(y), P(q), P(sc), None)


def test_rmsnorm_mxfp8_validation():
    assert _norm(n=0) == OK
    assert _norm(n=-1) == SHAPE
    assert _norm(d=4) == SHAPE
    assert _norm(d=(1 << 20) + 32) == SHAPE
    assert _norm(d=260) == UNSUP                        # d % 8
    assert _norm(d=264) == UNSUP                        # cast needs d % 32 == 0
    assert _norm(dtype=5) == UNSUP
    assert _norm(eps=-1.0) == ARG
    assert _norm(y=None, q=None, sc=None) == ARG         # nothing requested
    assert _norm(sc=None) == NULL                        # codes without scales
    assert _norm(x=None) == NULL
    assert _norm(q=0x40000004) == ALIGN
    assert _norm(y=A + 16) == ALIAS                      # partial overlap with x
    assert _norm(q=A + 64) == ALIAS                      # codes inside x
    assert _norm(sc=0x40000000 + 16 * 256 - 8) == ALIAS  # scales inside codes


def test_row_bound():
    """n >= 2^31 rows is rejected by every entry point before any launch, also where
    n * d is still within its own bound (the launch grids derive from n)."""
    big = 1 << 31
    assert _split(n=big) == SHAPE
    assert _split(n=big - 1, mixes=None) == NULL          # the bound itself passes
    assert _pre(n=big, d=8) == SHAPE
    assert _post(n=big, d=8) == SHAPE
    assert _mixes(n=big, d=8) == SHAPE
    assert _fused(n=big, d=8) == SHAPE


@pytest.mark.parametrize("fn", ["hc_pre", "hc_post", "hc_mixes", "hc_fused_step"])
def test_huge_shapes_rejected(fn):
    if fn == "hc_pre":
        assert _pre(n=1 << 40, d=1 << 20) == SHAPE
    elif fn == "hc_post":
        assert _post(n=1 << 40, d=1 << 20) == SHAPE
    elif fn == "hc_mixes":
        assert _mixes(n=1 << 40, d=1 << 20) == SHAPE
    else:
        assert _fused(n=1 << 40, d=1 << 20) == SHAPE


def test_generic_stream_count_spans():
    """Stream counts other than four size every span by hc: outputs that overlap at
    hc = 8 but would not at hc = 4 are rejected, and neighbouring buffers placed
    exactly hc-sized apart are accepted by validation (which then reaches the
    launch; only the error cases are run here)."""
    n = 16
    # split, hc = 8: pre is n*8*4 = 512 B; post placed 256 B after pre overlaps it
    assert _split(hc_=8, pre=0x40000000, post=0x40000000 + 256, comb=0x40010000,
                  mixes=0x50000000) == ALIAS
    # comb (n*64*4 = 4096 B at hc = 8) overlapping mixes' tail
    M8 = (2 + 8) * 8
    assert _split(hc_=8, mixes=0x50000000, pre=0x40000000, post=0x40001000,
                  comb=0x50000000 + n * M8 * 4 - 16) == ALIAS
    # pre, hc = 2: x is n*2*d elements; y right after x's 2 streams but inside 4 streams
    d = 256
    assert _pre(hc_=2, x=A, y=A + n * 2 * d * 2 - 16, d=d) == ALIAS
    # post, hc = 8: out partially overlapping the 8-stream residual
    assert hc.lib().hc_post(P(A), P(B), 1, P(C), P(C + 4096), n, 8, d, P(B + n * 8 * d * 2 - 32),
                            None) == ALIAS
    # mixes, hc = 3: the workspace must cover the unfused plan
    ws3 = hc.workspace_size(n, 3, d)
    assert hc.lib().hc_mixes(P(A), 1, n, 3, d, P(B), 1e-20, P(C), P(0x60000000), ws3 - 1, None) == WS


def test_fused_generic_validation():
    """hc_fused_step with hc = 5: null, workspace and alias rules use the unfused plan
    and hc-sized spans."""
    def fused(**kw):
        base = dict(res=A, pre_mix=0x50000000, fn=B, scale=C, base=C + 4096, n=16, d=256, dtype=1, iters=20,
                    y=0x60000000, pre=0x70000000, post=0x70001000, comb=0x70002000, mixes=None, ws=0x40000000,
                    ws_bytes=1 << 22, f_prev=None, post_prev=None, comb_prev=None, so=None)
        base.update(kw)
        return hc.lib().hc_fused_step(P(base["res"]), P(base["f_prev"]), P(base["post_prev"]),
                                      P(base["comb_prev"]), P(base["pre_mix"]), P(base["fn"]), P(base["scale"]),
                                      P(base["base"]), base["n"], 5, base["d"], base["dtype"], 1e-20,
                                      base["iters"], 1e-6, P(base["so"]), P(base["y"]), P(base["pre"]),
                                      P(base["post"]), P(base["comb"]), P(base["mixes"]), P(base["ws"]),
                                      base["ws_bytes"], None)
    assert fused(n=0) == OK
    assert fused(ws_bytes=hc.workspace_size(16, 5, 256) - 1) == WS
    assert fused(pre=None) == NULL
    assert fused(post=0x70000000 + 16 * 5 * 4 - 16) == ALIAS    # post overlaps pre's last 16 bytes
    assert fused(comb=0x70001000 + 16 * 5 * 4 - 16) == ALIAS    # comb overlaps post
    assert fused(f_prev=0x58000000, post_prev=0x59000000, comb_prev=0x59001000,
                 so=A + 16) == ALIAS                           # partial overlap with residual


def _fused_noalloc(res=A, pre_mix=0x50000000, fn=B, scale=C, base=C + 64, hc_=4, n=16, d=256, dtype=1,
                   iters=20, y=0x60000000, pre=0x70000000, post=0x70001000, comb=0x70002000, mixes=None):
    return hc.lib().hc_fused_step_noalloc(P(res), None, None, None, P(pre_mix), P(fn), P(scale), P(base), n, hc_, d,
                                          dtype, 1e-20, iters, 1e-6, None, P(y), P(pre), P(post), P(comb),
                                          P(mixes), None)


def test_fused_noalloc_validation():
    """The no-allocation variant validates like hc_fused_step (no workspace
    arguments) and refuses, before any HIP call, a size whose scratch need exceeds
    the static buffer (HC_ERR_SCRATCH)."""
    assert _fused_noalloc(n=0) == OK
    assert _fused_noalloc(iters=0) == ARG
    assert _fused_noalloc(pre=None) == NULL
    assert _fused_noalloc(scale=C + 2) == ALIGN
    assert _fused_noalloc(post=0x70000000 + 16 * 4 * 4 - 16) == ALIAS
    assert _fused_noalloc(n=1 << 40, d=1 << 20) == SHAPE
    assert hc.workspace_size(4096, 8, 5120) > 32 << 20
    assert _fused_noalloc(hc_=8, n=4096, d=5120) == -9
    # the largest four-stream token count at d = 5120 whose workspace fits the buffer
    lo, hi = 1, 1 << 22
    while lo < hi:
        mid = (lo + hi + 1) // 2
        lo, hi = (mid, hi) if hc.workspace_size(mid, 4, 5120) <= 32 << 20 else (lo, mid - 1)
    assert hc.workspace_size(lo + 1, 4, 5120) > 32 << 20
    assert _fused_noalloc(n=lo + 1, d=5120) == -9
    # within the buffer, validation passes and the first HIP call (no GPU here) fails
    assert _fused_noalloc(n=lo, d=5120, y=0x7000000000, pre=0x7100000000, post=0x7200000000,
                          comb=0x7300000000, pre_mix=0x7400000000, res=0x1000000000) == HIP


def _largest_accepted(hc_, d):
    """The largest token count hc_workspace_size accepts for (hc, d) (it returns 0
    for a shape the entry points reject)."""
    lo, hi = 0, (1 << 31) - 1
    while lo < hi:
        mid = (lo + hi + 1) // 2
        lo, hi = (mid, hi) if hc.workspace_size(mid, hc_, d) > 0 else (lo, mid - 1)
    return lo


@pytest.mark.parametrize("hc_,d", [(4, 8), (4, 5120), (4, 1 << 20), (2, 8), (8, 5120), (3, 1 << 20)])
def test_launch_grid_bounds(hc_, d):
    """Every kernel grid must fit a launch (2^32 - 1 work-items per dimension). The
    grids grow with the token count: with four streams the finalize takes 16 lanes
    per token and the collapse/expand a lane per 8 channels; other stream counts
    take a wave per token and per 512 channels. The documented limits follow, and
    the entry points reject the first size beyond them before any HIP call."""
    n = _largest_accepted(hc_, d)
    limit = (1 << 32) - 1
    grid = lambda lanes: -(-lanes // 256) * 256   # whole 256-thread workgroups
    if hc_ == 4:
        items = lambda m: max(grid(16 * m), grid(m * (d // 8)))
        assert n < 1 << 28 and n * d <= 1 << 35
    else:
        items = lambda m: grid(64 * m * -(-d // 512))
        assert n * -(-d // 512) < 1 << 26
    assert items(n) <= limit < items(n + 1)
    # the first rejected size, through every stream entry point (fake, far-apart pointers)
    far = [(k + 1) << 42 for k in range(10)]
    L = hc.lib()
    m = n + 1
    assert L.hc_pre(P(far[0]), 1, P(far[1]), m, hc_, d, P(far[2]), None) == SHAPE
    assert L.hc_post(P(far[0]), P(far[1]), 1, P(far[2]), P(far[3]), m, hc_, d, P(far[4]), None) == SHAPE
    assert L.hc_mixes(P(far[0]), 1, m, hc_, d, P(far[1]), 1e-20, P(far[2]), P(far[3]), 1 << 40, None) == SHAPE
    assert L.hc_fused_step(P(far[0]), None, None, None, P(far[1]), P(far[2]), P(far[3]), P(far[3] + 64), m, hc_, d,
                           1, 1e-20, 20, 1e-6, None, P(far[4]), P(far[5]), P(far[6]), P(far[7]), None, P(far[8]),
                           1 << 40, None) == SHAPE
    # at the largest accepted size, validation passes (the first HIP call fails: no GPU)
    assert L.hc_pre(P(far[0]), 1, P(far[1]), n, hc_, d, P(far[2]), None) == HIP


def test_split_grid_bound():
    """The split takes a lane per token with four streams and a wave per token with
    other stream counts."""
    L = hc.lib()
    big = (1 << 26) + 1
    assert L.hc_split_sinkhorn(P(1 << 42), P(2 << 42), P(3 << 42), big, 8, 20, 1e-6, P(4 << 42), P(5 << 42),
                               P(6 << 42), None) == SHAPE
    assert L.hc_split_sinkhorn(P(1 << 42), P(2 << 42), P(3 << 42), big, 4, 20, 1e-6, P(4 << 42), P(5 << 42),
                               P(6 << 42), None) == HIP
