"""GPU parity for stream counts other than four (1 <= hc <= 8) and for Sinkhorn
round counts other than 20, through the C ABI, against the oracle on the same
seeded inputs.

The page's split kernel and Block are written for any stream count; the library
runs four streams on its single-pass kernels and other counts on one kernel per
step. Sizes leave partial 64-token tiles and partial 64-column tiles of the
flattened hc*d axis, and reach the smallest width d = 8. Tolerances and the
comparison rule are in tests/parity.py.
"""
import pytest
import torch

import hc_inputs
import hyper_connection_residual_mixes_amd as hc
import oracle
from parity import TOL_BF16, TOL_F32, check, rho_for

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
HCS = [1, 2, 3, 5, 6, 7, 8]   # the projection's column-tile counts R = ceil((2+hc)hc / 16): 1, 3, 4, 5


def to_dev(t):
    return t.to(DEV) if isinstance(t, torch.Tensor) else tuple(to_dev(u) for u in t)


def sync():
    torch.cuda.synchronize()


# -------------------------------------------------------------------- split
@pytest.mark.parametrize("hc_", HCS + [4])
@pytest.mark.parametrize("n,iters", [(1, 20), (257, 1), (300, 7), (1000, 20)])
def test_split(hc_, n, iters):
    g = hc_inputs.generator(30 + hc_)
    M = (2 + hc_) * hc_
    m = hc_inputs.normal(g, (n, M), 2.0)
    s = torch.rand(3, generator=g) * 1.5 + 0.5
    b = hc_inputs.normal(g, (M,), 0.1)
    ref = oracle.hc_split_sinkhorn(m, s, b, hc_mult=hc_, sinkhorn_iters=iters)
    got = hc.hc_split_sinkhorn(*to_dev((m, s, b)), hc_mult=hc_, sinkhorn_iters=iters)
    sync()
    for name, gg, r in zip(("pre", "post", "comb"), got, ref):
        check(f"hc={hc_} n={n} it={iters} {name}", gg, r, TOL_F32, rho=1.0)


@pytest.mark.parametrize("hc_", HCS)
def test_split_large_eps(hc_):
    """eps = 0.3, so that where it enters each normalisation shows far above the
    tolerance."""
    g = hc_inputs.generator(60 + hc_)
    M = (2 + hc_) * hc_
    m = hc_inputs.normal(g, (300, M), 2.0)
    s = torch.rand(3, generator=g) * 1.5 + 0.5
    b = hc_inputs.normal(g, (M,), 0.1)
    ref = oracle.hc_split_sinkhorn(m, s, b, hc_mult=hc_, sinkhorn_iters=5, eps=0.3)
    got = hc.hc_split_sinkhorn(*to_dev((m, s, b)), hc_mult=hc_, sinkhorn_iters=5, eps=0.3)
    sync()
    for name, gg, r in zip(("pre", "post", "comb"), got, ref):
        check(f"hc={hc_} eps=0.3 {name}", gg, r, TOL_F32, rho=1.0)


# ------------------------------------------------------------- pre / post
CASES = [(torch.float32, 37, 264), (torch.bfloat16, 37, 264), (torch.bfloat16, 1, 8),
         (torch.bfloat16, 64, 5120)]


def _streams_case(hc_, dtype, n, d, seed):
    g = hc_inputs.generator(seed)
    x = hc_inputs.streams(g, n, hc_, d, dtype, outlier_frac=0.1)
    f = hc_inputs.sublayer_output(g, n, d, dtype)
    w = torch.rand(n, hc_, generator=g)
    post = torch.rand(n, hc_, generator=g) * 2
    comb = torch.rand(n, hc_, hc_, generator=g)
    return x, f, w, post, comb


@pytest.mark.parametrize("hc_", HCS)
@pytest.mark.parametrize("dtype,n,d", CASES)
def test_pre_and_post(hc_, dtype, n, d):
    x, f, w, post, comb = _streams_case(hc_, dtype, n, d, seed=40 + hc_)
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    xd, fd, wd, pd, cd = to_dev((x, f, w, post, comb))
    y = hc.hc_pre(xd, wd)
    out = hc.hc_post(fd, xd, pd, cd)
    sync()
    check(f"hc={hc_} pre {dtype} {n}x{d}", y, oracle.hc_pre(x, w), tol)
    check(f"hc={hc_} post {dtype} {n}x{d}", out, oracle.hc_post(f, x, post, comb), tol)
    hc.hc_post(fd, xd, pd, cd, out=xd)          # exact in-place
    sync()
    assert torch.equal(xd.cpu(), out.cpu())


# ------------------------------------------------------------------- mixes
@pytest.mark.parametrize("hc_", HCS)
@pytest.mark.parametrize("dtype,n,d", [(torch.float32, 16, 256), (torch.float32, 37, 264),
                                       (torch.bfloat16, 37, 264), (torch.bfloat16, 70, 5120),
                                       (torch.bfloat16, 3, 8), (torch.float32, 130, 8),
                                       (torch.bfloat16, 300, 264)])
def test_mixes(hc_, dtype, n, d):
    g = hc_inputs.generator(50 + hc_)
    fn, _, _ = hc_inputs.mix_params(g, hc_, d, "ones")
    x = hc_inputs.streams(g, n, hc_, d, dtype, outlier_frac=0.1)
    ref = oracle.hc_mixes(x, fn)
    xd, fnd = to_dev((x, fn))
    ws = torch.full((hc.workspace_size(n, hc_, d),), 255, dtype=torch.uint8, device=DEV)  # NaN bytes
    got = hc.hc_mixes(xd, fnd, workspace=ws)
    sync()
    assert got.shape == (n, (2 + hc_) * hc_)
    check(f"hc={hc_} mixes {dtype} {n}x{d}", got, ref, TOL_F32)


# ----------------------------------------------------------- fused / block
def _block_inputs(hc_, dtype, n, d, seed):
    g = hc_inputs.generator(seed)
    mode = "ones" if dtype == torch.float32 else "uniform"
    attn = hc_inputs.mix_params(g, hc_, d, mode)
    ffn = hc_inputs.mix_params(g, hc_, d, mode)
    x = hc_inputs.streams(g, n, hc_, d, dtype, outlier_frac=0.05)
    f_attn = hc_inputs.sublayer_output(g, n, d, dtype)
    f_ffn = hc_inputs.sublayer_output(g, n, d, dtype)
    prev = hc_inputs.previous_call(g, n, hc_)
    return x, attn, ffn, f_attn, f_ffn, prev


@pytest.mark.parametrize("hc_,iters", [(1, 20), (2, 20), (3, 5), (4, 5), (5, 20), (6, 20), (7, 3), (8, 20),
                                       (8, 1)])
@pytest.mark.parametrize("dtype,n,d", [(torch.float32, 16, 256), (torch.bfloat16, 37, 264),
                                       (torch.bfloat16, 64, 5120), (torch.bfloat16, 5, 8)])
def test_block(hc_, iters, dtype, n, d):
    """Attention boundary, FFN boundary (expand + coefficients + collapse with the
    attention's pre), FFN expand. The FFN coefficients come from the rounded streams
    x1, so for bf16 they are held to the bf16 tolerance (as for four streams)."""
    x, attn, ffn, f_attn, f_ffn, prev = _block_inputs(hc_, dtype, n, d, seed=60 + hc_)
    pi = oracle.hc_split_sinkhorn(*prev, hc_mult=hc_)[0]
    ref = oracle.block(x, pi, attn, ffn, f_attn, f_ffn, sinkhorn_iters=iters)
    got = hc.block(*to_dev((x, pi)), to_dev(attn), to_dev(ffn), *to_dev((f_attn, f_ffn)),
                   sinkhorn_iters=iters)
    sync()
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    for k in ("preA", "postA", "combA"):
        check(f"hc={hc_} {k}", got[k], ref[k], TOL_F32, rho=1.0)
    for k in ("yA", "x1", "yF", "x2"):
        check(f"hc={hc_} {k}", got[k], ref[k], tol)
    for k in ("preF", "postF", "combF"):
        check(f"hc={hc_} {k}", got[k], ref[k], tol, rho=1.0)


@pytest.mark.parametrize("hc_", HCS)
def test_fused_exact_inputs_and_in_place(hc_):
    """The fused step on streams both sides receive exactly: mixes and coefficients
    within 1e-5; then with the expand step written in place over the residual."""
    dtype, n, d = torch.bfloat16, 64, 5120
    x, attn, ffn, f_attn, _, prev = _block_inputs(hc_, dtype, n, d, seed=70 + hc_)
    pi = oracle.hc_split_sinkhorn(*prev, hc_mult=hc_)[0]
    ref = oracle.fused_step(x, *ffn, pre_mix=pi)
    got = hc.hc_fused_step(*to_dev((x,)), *to_dev(ffn), pre_mix=to_dev(pi), want_mixes=True)
    sync()
    for k in ("mixes", "pre", "post", "comb"):
        check(f"hc={hc_} {k}", got[k], ref[k], TOL_F32, rho=rho_for(k))
    check(f"hc={hc_} y", got["y"], ref["y"], TOL_BF16)
    post, comb = got["post"], got["comb"]
    ref2 = oracle.fused_step(x, *attn, pre_mix=pi, f_prev=f_attn, post_prev=post.cpu(), comb_prev=comb.cpu())
    xd = x.to(DEV)
    got2 = hc.hc_fused_step(xd, *to_dev(attn), pre_mix=to_dev(pi), f_prev=f_attn.to(DEV), post_prev=post,
                            comb_prev=comb, streams_out=xd)
    sync()
    check(f"hc={hc_} streams (in place)", xd, ref2["streams"], TOL_BF16)
    check(f"hc={hc_} y after expand", got2["y"], ref2["y"], TOL_BF16)


@pytest.mark.parametrize("hc_,n,iters", [(2, 4096, 20), (2, 37, 7), (2, 1, 1), (8, 300, 20), (8, 5, 3)])
def test_fused_split_same_bits_as_split(hc_, n, iters):
    """The split fused into the finalize (four lanes per token at two streams, the
    butterfly at eight) gives the same bits as hc_split_sinkhorn on the mixes the
    fused step returns: both run the same fp32 steps, with every lane of a comb row
    or column adding the same numbers (no contraction of a lane's own product)."""
    dtype, d = torch.bfloat16, 264
    x, attn, _, _, _, prev = _block_inputs(hc_, dtype, n, d, seed=90 + hc_)
    pi = oracle.hc_split_sinkhorn(*prev, hc_mult=hc_)[0]
    _, scale, base = attn
    got = hc.hc_fused_step(*to_dev((x,)), *to_dev(attn), pre_mix=to_dev(pi), sinkhorn_iters=iters,
                           want_mixes=True)
    pre, post, comb = hc.hc_split_sinkhorn(got["mixes"], *to_dev((scale, base)), hc_mult=hc_,
                                           sinkhorn_iters=iters)
    sync()
    assert torch.equal(got["pre"], pre)
    assert torch.equal(got["post"], post)
    assert torch.equal(got["comb"], comb)


@pytest.mark.parametrize("hc_", [2, 8])
def test_block_full_size_sampled(hc_):
    """The prefill block at two and eight streams (4096 tokens x 5120 bf16, 1% x50
    outliers: the inputs and launch configuration the benchmark times). Every step is
    per token, so the oracle runs on 48 sampled tokens only; those tokens of every
    output are compared, with the tolerances of test_block."""
    w = hc_inputs.Workload(f"prefill_hc{hc_}", 1, 4096, 5120, torch.bfloat16, hc=hc_)
    inp = hc_inputs.block_inputs(w, seed=0, outlier_frac=0.01)
    pi = oracle.hc_split_sinkhorn(*inp["prev"], hc_mult=hc_)[0]
    got = hc.block(*to_dev((inp["x"], pi)), to_dev(inp["attn"]), to_dev(inp["ffn"]),
                   *to_dev((inp["f_attn"], inp["f_ffn"])))
    sync()
    sample = torch.randperm(w.n, generator=hc_inputs.generator(11))[:48].sort().values
    print(f"  hc={hc_} full-size block, sampled tokens {sample[:4].tolist()}...", flush=True)
    ref = oracle.block(inp["x"][sample], pi[sample], inp["attn"], inp["ffn"], inp["f_attn"][sample],
                       inp["f_ffn"][sample])
    rows = lambda t: t[sample.to(t.device)].cpu()
    for k in ("preA", "postA", "combA"):
        check(f"hc={hc_} {k} (sampled)", rows(got[k]), ref[k], TOL_F32, rho=1.0)
    for k in ("yA", "x1", "yF", "x2", "preF", "postF", "combF"):
        check(f"hc={hc_} {k} (sampled)", rows(got[k]), ref[k], TOL_BF16, rho=rho_for(k))


@pytest.mark.parametrize("hc_,dtype,n,d", [(8, torch.bfloat16, 820, 5120), (2, torch.float32, 2049, 4096)])
def test_post_streamed_output(hc_, dtype, n, d):
    """64 MiB and more of expand output are written with non-temporal stores."""
    x, f, _, post, comb = _streams_case(hc_, dtype, n, d, seed=80 + hc_)
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    xd, fd, pd, cd = to_dev((x, f, post, comb))
    out = hc.hc_post(fd, xd, pd, cd)
    sync()
    check(f"hc={hc_} post {dtype} {n}x{d} (streamed)", out, oracle.hc_post(f, x, post, comb), tol)
    hc.hc_post(fd, xd, pd, cd, out=xd)          # exact in-place
    sync()
    assert torch.equal(xd.cpu(), out.cpu())
