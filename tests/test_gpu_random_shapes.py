"""GPU parity of the whole block (attention boundary, FFN boundary, FFN expand) on
seeded random configurations against the oracle.

The configurations are drawn once from a fixed seed: stream counts 1..8 (four
included, which runs the single-pass kernels), 1..300 tokens, widths d = 8k up
to 2400 (ragged against the 64-token tiles, 64-channel steps and 64-column
tiles), both stream dtypes and 1..25 Sinkhorn rounds; four random bf16 blocks of 1024..3000 tokens (the
128-token sweep); and the widest supported stream, d = 2^20, at a few tokens. Tolerances as in the block tests.
"""
import random

import pytest
import torch

import hc_inputs
import hyper_connection_residual_mixes_amd as hc
import oracle
from parity import TOL_BF16, TOL_F32, check

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _cases(count=24, seed=2024):
    rng = random.Random(seed)
    out = []
    for i in range(count):
        hc_ = 4 if i % 4 == 0 else rng.randint(1, 8)
        n = rng.choice([1, 2, 3, rng.randint(4, 63), rng.randint(64, 300)])
        d = 8 * rng.choice([1, 2, rng.randint(3, 40), rng.randint(41, 300)])
        dtype = rng.choice([torch.float32, torch.bfloat16])
        iters = rng.choice([1, 2, 20, rng.randint(3, 25)])
        out.append((hc_, n, d, dtype, iters, 100 + i))
    return out


@pytest.mark.parametrize("hc_,n,d,dtype,iters,seed", _cases())
def test_block_random_shape(hc_, n, d, dtype, iters, seed):
    _block_case(hc_, n, d, dtype, iters, seed)


def _wide_cases(count=4, seed=77):
    rng = random.Random(seed)
    return [(rng.randint(1024, 3000), 8 * rng.randint(1, 300), 200 + i) for i in range(count)]


# Four bf16 streams from 1024 tokens on run the 128-token sweep: seeded random token
# counts (ragged against 128) and widths (ragged against 64-channel steps).
@pytest.mark.parametrize("n,d,seed", _wide_cases())
def test_block_random_wide_sweep(n, d, seed):
    _block_case(4, n, d, torch.bfloat16, 20, seed)


# The widest supported stream, d = 2^20: the largest per-lane and per-row byte
# offsets the kernels form (the single-pass sweeps, the fp32 pass, the generic bf16
# projection and the wide projection of five to eight streams, whose weight rows
# are then 2^23 floats), a few tokens each so the oracle stays within seconds.
@pytest.mark.parametrize("hc_,n,dtype,seed", [(4, 3, torch.bfloat16, 900), (4, 2, torch.float32, 901),
                                              (2, 3, torch.bfloat16, 902), (2, 3, torch.float32, 903),
                                              (8, 2, torch.bfloat16, 904), (5, 3, torch.bfloat16, 905)])
def test_block_max_width(hc_, n, dtype, seed):
    _block_case(hc_, n, 1 << 20, dtype, 20, seed)


def _block_case(hc_, n, d, dtype, iters, seed):
    g = hc_inputs.generator(seed)
    mode = "ones" if dtype == torch.float32 else "uniform"
    attn = hc_inputs.mix_params(g, hc_, d, mode)
    ffn = hc_inputs.mix_params(g, hc_, d, mode)
    x = hc_inputs.streams(g, n, hc_, d, dtype, outlier_frac=0.05)
    f_attn = hc_inputs.sublayer_output(g, n, d, dtype)
    f_ffn = hc_inputs.sublayer_output(g, n, d, dtype)
    pi = oracle.hc_split_sinkhorn(*hc_inputs.previous_call(g, n, hc_), hc_mult=hc_)[0]
    ref = oracle.block(x, pi, attn, ffn, f_attn, f_ffn, sinkhorn_iters=iters)
    dev = lambda t: t.to(DEV) if isinstance(t, torch.Tensor) else tuple(u.to(DEV) for u in t)
    got = hc.block(dev(x), dev(pi), dev(attn), dev(ffn), dev(f_attn), dev(f_ffn), sinkhorn_iters=iters)
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    name = f"hc={hc_} n={n} d={d} {dtype} it={iters}"
    for k in ("preA", "postA", "combA"):
        check(f"{name} {k}", got[k], ref[k], TOL_F32, rho=1.0)
    for k in ("yA", "x1", "yF", "x2"):
        check(f"{name} {k}", got[k], ref[k], tol)
    for k in ("preF", "postF", "combF"):
        check(f"{name} {k}", got[k], ref[k], tol, rho=1.0)
