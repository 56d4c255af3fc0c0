"""hc_fused_step_noalloc (the fused boundary on the library's static device
scratch) against hc_fused_step (the same boundary on a caller workspace).

Both run the same kernels, so every output must be identical bit for bit, which
is stronger than the parity bar (1e-5 for fp32 results, 2e-2 for bf16 streams).
Consecutive calls share the scratch: the second call here is smaller than the
first, with a different slice plan, so stale partial rows of the first call would
show up in its results. A size beyond the scratch is refused before any launch.
"""
import pytest
import torch

import hc_inputs
import hyper_connection_residual_mixes_amd as hc
from parity import TOL_BF16, TOL_F32, check, rho_for

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def to_dev(t):
    return t.to(DEV) if isinstance(t, torch.Tensor) else tuple(to_dev(u) for u in t)


def _case(n, d, dtype, hc_mult=4, expand=True, seed=31):
    w = hc_inputs.Workload(f"noalloc_{n}x{d}", 1, n, d, dtype, hc=hc_mult)
    inp = hc_inputs.block_inputs(w, seed=seed, device=DEV, outlier_frac=0.01, scale_mode="uniform")
    g = hc_inputs.generator(seed + 1, DEV)
    kw = dict(pre_mix=torch.rand(n, hc_mult, generator=g, device=DEV), want_mixes=True)
    if expand:
        kw.update(f_prev=inp["f_attn"], post_prev=torch.rand(n, hc_mult, generator=g, device=DEV) * 2,
                  comb_prev=torch.rand(n, hc_mult, hc_mult, generator=g, device=DEV))
    return inp["x"], inp["ffn"], kw


def _compare(label, x, params, kw):
    ref = hc.hc_fused_step(x, *params, **kw)
    got = hc.hc_fused_step_noalloc(x, *params, **kw)
    torch.cuda.synchronize()
    tol = TOL_F32 if x.dtype == torch.float32 else TOL_BF16
    for k in ("streams", "y", "mixes", "pre", "post", "comb"):
        kt = TOL_F32 if k in ("mixes", "pre", "post", "comb") else tol
        check(f"{label} {k}", got[k], ref[k], kt, rho=rho_for(k))
        assert torch.equal(got[k], ref[k]), f"{label} {k}: not bit-identical to hc_fused_step"


def test_noalloc_two_calls_second_smaller():
    """The prefill FFN boundary (4096 tokens, 128-token sweep, 8 slices), then a
    smaller attention boundary (1031 x 1288: fewer tokens, another slice plan),
    each against hc_fused_step on the same inputs."""
    x, p, kw = _case(4096, 5120, torch.bfloat16)
    _compare("prefill FFN boundary", x, p, kw)
    x, p, kw = _case(1031, 1288, torch.bfloat16, expand=False, seed=32)
    _compare("1031x1288 attention boundary", x, p, kw)


def test_noalloc_other_paths():
    """The 64-token sweep (decode size), the fp32 pass and a stream count other
    than four (unfused kernels: partial rows and mixes in the scratch), in turn."""
    for n, d, dtype, h in ((64, 5120, torch.bfloat16, 4), (37, 264, torch.float32, 4), (300, 512, torch.bfloat16, 8),
                           (5, 64, torch.bfloat16, 2)):
        x, p, kw = _case(n, d, dtype, hc_mult=h, seed=33 + n)
        _compare(f"hc={h} {n}x{d} {dtype}", x, p, kw)


def test_noalloc_refuses_sizes_beyond_the_scratch():
    """Eight streams at 4096 x 5120 need 36.7 MB of scratch, above the 32 MiB the
    library holds: refused with HC_ERR_SCRATCH before anything is enqueued."""
    n, d, h = 4096, 5120, 8
    assert hc.workspace_size(n, h, d) > 32 << 20
    x = torch.zeros(n, h, d, dtype=torch.bfloat16, device=DEV)
    M = (2 + h) * h
    params = (torch.zeros(M, h * d, device=DEV), torch.ones(3, device=DEV), torch.zeros(M, device=DEV))
    with pytest.raises(hc.HCError) as ei:
        hc.hc_fused_step_noalloc(x, *params, pre_mix=torch.zeros(n, h, device=DEV))
    assert ei.value.status == -9
