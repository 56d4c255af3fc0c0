"""Per-step parity with teacher-forced inputs for the boundaries that expand.

A fused boundary with the expand step first writes the new streams x1 (rounded to
the stream dtype), then computes this sublayer's coefficients from the ROUNDED x1
and collapses x1 ("Block" page, code section: hc_post returns the streams in the
sublayer output's dtype, and the next hc_mixes flattens and widens exactly those
values). Chained against the oracle's own x1, an element that the two sides round
to neighbouring bf16 values moves the mixes by ~1e-5, so the block tests can hold
those coefficients only to the bf16 tolerance.

Here the oracle is fed the GPU's own x1 instead (teacher forcing), so everything
computed after the expand is held to the fp32 tolerance 1e-5: mixes, pre, post,
comb. The expand itself is checked on identical inputs (the oracle's expand of the
same streams, sublayer output and previous coefficients), and the collapse of the
GPU's x1 is held to the stream tolerance. This catches a projection of the
unrounded expanded values (a shift of ~1e-4 in the mixes) and any weight term
dropped in the expand instances of the sweeps.

Cases: every instance of the bf16 sweep with the expand (64-token and 128-token
groups, with and without the collapse), the fp32 pass, the full decode and
prefill FFN boundaries, ragged token counts and widths; for five to eight streams,
the boundary with the wide (256-token) projection after the expand.
"""
import pytest
import torch

import hc_inputs
import hyper_connection_residual_mixes_amd as hc
import oracle
from parity import TOL_BF16, TOL_F32, check, rho_for

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def to_dev(t):
    return t.to(DEV) if isinstance(t, torch.Tensor) else tuple(to_dev(u) for u in t)


def teacher_forced_boundary(label, x, params, f_prev, post_prev, comb_prev, pi=None):
    """Runs the GPU boundary with the expand on (x, f_prev, post_prev, comb_prev),
    then checks its x1 against the oracle's expand of the same inputs and every
    later output against the oracle run on the GPU's x1. pi None: no collapse."""
    tol_s = TOL_F32 if x.dtype == torch.float32 else TOL_BF16
    got = hc.hc_fused_step(*to_dev((x,)), *to_dev(params), pre_mix=None if pi is None else to_dev(pi),
                           f_prev=to_dev(f_prev), post_prev=to_dev(post_prev), comb_prev=to_dev(comb_prev),
                           want_mixes=True, want_y=pi is not None)
    torch.cuda.synchronize()
    x1 = got["streams"].cpu()
    check(f"{label} x1 (same inputs)", x1, oracle.hc_post(f_prev, x, post_prev, comb_prev), tol_s)
    ref = oracle.fused_step(x1, *params, pre_mix=pi if pi is not None else torch.zeros(x.shape[0], x.shape[1]))
    for k in ("mixes", "pre", "post", "comb"):
        check(f"{label} {k} (GPU x1)", got[k], ref[k], TOL_F32, rho=rho_for(k))
    if pi is not None:
        check(f"{label} y (GPU x1)", got["y"], ref["y"], tol_s)
    else:
        assert got["y"] is None
    return got


def _block_boundary(inp):
    """The FFN boundary of a block: the oracle's attention coefficients (post, comb,
    pre) are the previous-sublayer inputs both sides receive."""
    x = inp["x"]
    _, preA, postA, combA = oracle.hc_mixes_split(x, *inp["attn"], hc_mult=x.shape[-2])
    return x, inp["ffn"], inp["f_attn"], postA, combA, preA


@pytest.mark.parametrize("which", ["decode", "prefill"])
def test_ffn_boundary_full(which):
    """The full decode (64 tokens: 64-token sweep) and prefill (4096 tokens, 1% x50
    outliers: 128-token sweep, the benchmark's launch configuration) FFN boundaries."""
    inp = hc_inputs.decode(seed=0) if which == "decode" else hc_inputs.prefill(seed=0)
    x, ffn, f, post, comb, pi = _block_boundary(inp)
    teacher_forced_boundary(which, x, ffn, f, post, comb, pi)


@pytest.mark.parametrize("dtype,n,d", [(torch.bfloat16, 1031, 1288), (torch.bfloat16, 130, 5120),
                                       (torch.bfloat16, 37, 264), (torch.bfloat16, 1, 8),
                                       (torch.bfloat16, 1024, 64), (torch.float32, 37, 264),
                                       (torch.float32, 70, 1032)])
@pytest.mark.parametrize("collapse", [True, False])
def test_ragged(dtype, n, d, collapse):
    """Ragged token counts (partial 64- and 128-token groups) and widths (a partial
    last 64-channel step, a single step), with and without the collapse."""
    w = hc_inputs.Workload(f"tf_{n}x{d}", 1, n, d, dtype)
    inp = hc_inputs.block_inputs(w, seed=13, outlier_frac=0.05, scale_mode="uniform")
    x, ffn, f, post, comb, pi = _block_boundary(inp)
    teacher_forced_boundary(f"{dtype} {n}x{d}", x, ffn, f, post, comb, pi if collapse else None)


def test_in_place_expand():
    """The in-place expand (streams_out == residual) of a 128-token sweep: the
    coefficients equal those of the out-of-place call bit for bit, so they inherit
    its teacher-forced parity."""
    w = hc_inputs.Workload("tf_inplace", 1, 1100, 640, torch.bfloat16)
    inp = hc_inputs.block_inputs(w, seed=14, outlier_frac=0.02, scale_mode="uniform")
    x, ffn, f, post, comb, pi = _block_boundary(inp)
    got = teacher_forced_boundary("out of place", x, ffn, f, post, comb, pi)
    xd = to_dev(x)
    got2 = hc.hc_fused_step(xd, *to_dev(ffn), pre_mix=to_dev(pi), f_prev=to_dev(f), post_prev=to_dev(post),
                            comb_prev=to_dev(comb), streams_out=xd, want_mixes=True)
    torch.cuda.synchronize()
    assert torch.equal(xd.cpu(), got["streams"].cpu())
    for k in ("y", "mixes", "pre", "post", "comb"):
        assert torch.equal(got2[k].cpu(), got[k].cpu()), k


@pytest.mark.parametrize("hc_", [5, 6, 7, 8])
@pytest.mark.parametrize("n,d", [(130, 1288), (64, 5120), (3, 8), (600, 264)])
@pytest.mark.parametrize("collapse", [True, False])
def test_generic_expand_boundary(hc_, n, d, collapse):
    """Five to eight bf16 streams: the expand, then the wide projection of the rounded
    x1. Ragged token counts (partial 256-token tiles) and widths (a partial last
    64-channel block; d = 8 a single partial block)."""
    w = hc_inputs.Workload(f"tf_hc{hc_}_{n}x{d}", 1, n, d, torch.bfloat16, hc=hc_)
    inp = hc_inputs.block_inputs(w, seed=15 + hc_, outlier_frac=0.05, scale_mode="uniform")
    x, ffn, f, post, comb, pi = _block_boundary(inp)
    teacher_forced_boundary(f"hc={hc_} {n}x{d}", x, ffn, f, post, comb, pi if collapse else None)


def test_generic_expand_boundary_full_size_in_place():
    """Eight streams at the prefill size (4096 tokens x 5120, 1% x50 outliers: the
    launch configuration the benchmark times), teacher-forced on 48 sampled tokens;
    then the same call in place over the residual, bit-identical."""
    w = hc_inputs.Workload("tf_hc8_prefill", 1, 4096, 5120, torch.bfloat16, hc=8)
    inp = hc_inputs.block_inputs(w, seed=16, outlier_frac=0.01)
    # previous coefficients from the oracle's split of the drawn logits (no projection of 4096 tokens)
    pi, post, comb = oracle.hc_split_sinkhorn(*inp["prev"], hc_mult=8)
    x, ffn, f = inp["x"], inp["ffn"], inp["f_attn"]
    got = hc.hc_fused_step(*to_dev((x,)), *to_dev(ffn), pre_mix=to_dev(pi), f_prev=to_dev(f),
                           post_prev=to_dev(post), comb_prev=to_dev(comb), want_mixes=True)
    torch.cuda.synchronize()
    sample = torch.randperm(w.n, generator=hc_inputs.generator(12))[:48].sort().values
    x1 = got["streams"][sample.to(DEV)].cpu()
    check("hc=8 prefill x1 (sampled, same inputs)", x1,
          oracle.hc_post(f[sample], x[sample], post[sample], comb[sample]), TOL_BF16)
    ref = oracle.fused_step(x1, *ffn, pre_mix=pi[sample])
    for k in ("mixes", "pre", "post", "comb"):
        check(f"hc=8 prefill {k} (sampled, GPU x1)", got[k][sample.to(DEV)].cpu(), ref[k], TOL_F32,
              rho=rho_for(k))
    check("hc=8 prefill y (sampled, GPU x1)", got["y"][sample.to(DEV)].cpu(), ref["y"], TOL_BF16)
    xd = to_dev(x)
    got2 = hc.hc_fused_step(xd, *to_dev(ffn), pre_mix=to_dev(pi), f_prev=to_dev(f), post_prev=to_dev(post),
                            comb_prev=to_dev(comb), streams_out=xd, want_mixes=True)
    torch.cuda.synchronize()
    assert torch.equal(xd.cpu(), got["streams"].cpu())
    for k in ("y", "mixes", "pre", "post", "comb"):
        assert torch.equal(got2[k].cpu(), got[k].cpu()), k
