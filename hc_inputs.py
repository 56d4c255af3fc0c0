"""Seeded synthetic inputs for the hyper-connection residual mix.

This module is shared by the tests, the benchmark and the smoke check; it feeds the
same tensors to the HIP library and to the CPU oracle. It draws random numbers
only: none of the method's arithmetic lives here.

The shapes and distributions follow the workloads of the DeepSeek-V4.1 model the
pages describe (4 streams of width 5120, fp32 mix parameters, bf16 streams) at the
sizes listed below; there is no public dataset for this computation, so seeded
normal draws stand in for activations and trained weights.

Every draw comes from one ``torch.Generator`` seeded with ``seed`` and is taken in
the order written in each function, so a config and seed always give the same
tensors. ``N(0, s)`` below means standard deviation ``s``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

HC = 4


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq: int
    d: int
    dtype: torch.dtype
    hc: int = HC

    @property
    def n(self) -> int:
        return self.batch * self.seq


TINY = Workload("tiny_fp32_T16_d256", 1, 16, 256, torch.float32)
DECODE = Workload("decode_B64_T1_d5120_bf16", 64, 1, 5120, torch.bfloat16)
PREFILL = Workload("prefill_B1_T4096_d5120_bf16", 1, 4096, 5120, torch.bfloat16)
LONG_PREFILL = Workload("long_prefill_B2_T32768_d5120_bf16", 2, 32768, 5120, torch.bfloat16)
STRESS_ROWS = 1_048_576


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(g, shape, std=1.0, device="cpu"):
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * std


def mix_params(g, hc: int, d: int, scale_mode: str, device="cpu"):
    """One stream-weight instance: hc_fn [(2+hc)hc, hc*d] ~ N(0, 1/sqrt(hc*d)),
    hc_base [(2+hc)hc] ~ N(0, 0.1), hc_scale [3] = ones ("ones") or ~ U(0.5, 2) ("uniform")."""
    M = (2 + hc) * hc
    D = hc * d
    fn = normal(g, (M, D), 1.0 / math.sqrt(D), device)
    base = normal(g, (M,), 0.1, device)
    if scale_mode == "ones":
        scale = torch.ones(3, dtype=torch.float32, device=device)
    elif scale_mode == "uniform":
        scale = torch.rand(3, generator=g, device=device, dtype=torch.float32) * 1.5 + 0.5
    else:
        raise ValueError(scale_mode)
    return fn, scale, base


def streams(g, n: int, hc: int, d: int, dtype, outlier_frac=0.0, outlier_scale=50.0, device="cpu"):
    """x [n, hc, d] ~ N(0, 1); a fraction of token rows (a row = one token's whole
    [hc, d] block, picked without replacement) is multiplied by ``outlier_scale`` in
    fp32 before the cast to ``dtype``."""
    x = normal(g, (n, hc, d), 1.0, device)
    n_out = int(round(outlier_frac * n))
    if n_out:
        rows = torch.randperm(n, generator=g, device=device)[:n_out]
        x[rows] *= outlier_scale
    return x.to(dtype)


def sublayer_output(g, n: int, d: int, dtype, device="cpu"):
    """Stand-in for a sublayer body's output: [n, d] ~ N(0, 1) in ``dtype``."""
    return normal(g, (n, d), 1.0, device).to(dtype)


def previous_call(g, n: int, hc: int, device="cpu"):
    """Inputs of the split step of a PREVIOUS sublayer, whose pre weights become this
    sublayer's collapse weights: logits [n, (2+hc)hc] ~ N(0, 1), scale ~ U(0.5, 2),
    base ~ N(0, 0.1). The caller runs its own split on them."""
    M = (2 + hc) * hc
    logits = normal(g, (n, M), 1.0, device)
    scale = torch.rand(3, generator=g, device=device, dtype=torch.float32) * 1.5 + 0.5
    base = normal(g, (M,), 0.1, device)
    return logits, scale, base


def block_inputs(w: Workload, seed: int = 0, device="cpu", outlier_frac=0.0, scale_mode=None):
    """Inputs of one block (attention + FFN boundary) of workload ``w``.

    Draw order: attention params, FFN params, streams, f_attn, f_ffn, previous call.
    """
    g = generator(seed, device)
    if scale_mode is None:
        scale_mode = "ones" if w.dtype == torch.float32 else "uniform"
    attn = mix_params(g, w.hc, w.d, scale_mode, device)
    ffn = mix_params(g, w.hc, w.d, scale_mode, device)
    x = streams(g, w.n, w.hc, w.d, w.dtype, outlier_frac, device=device)
    f_attn = sublayer_output(g, w.n, w.d, w.dtype, device)
    f_ffn = sublayer_output(g, w.n, w.d, w.dtype, device)
    prev = previous_call(g, w.n, w.hc, device)
    return dict(workload=w, attn=attn, ffn=ffn, x=x, f_attn=f_attn, f_ffn=f_ffn, prev=prev)


def tiny(seed: int = 0):
    """B=1, T=16, 4 streams, d=256, fp32 streams; hc_scale = [1, 1, 1]."""
    return block_inputs(TINY, seed)


def decode(seed: int = 0, device="cpu"):
    """B=64, T=1, d=5120, bf16 streams, two mix-parameter sets with scale ~ U(0.5, 2)."""
    return block_inputs(DECODE, seed, device)


def prefill(seed: int = 0, device="cpu"):
    """B=1, T=4096, d=5120, bf16 streams with 1% of token rows scaled by 50."""
    return block_inputs(PREFILL, seed, device, outlier_frac=0.01)


def stress(seed: int = 0, rows: int = STRESS_ROWS, hc: int = HC, device="cpu"):
    """Split stage only: logits [rows, (2+hc)hc] ~ N(0, 3); in 5% of rows (picked
    without replacement) one comb logit, at an index drawn uniformly from the comb
    block [2hc, (2+hc)hc), is raised by 40. hc_scale = [1,1,1], hc_base = 0."""
    g = generator(seed, device)
    M = (2 + hc) * hc
    logits = normal(g, (rows, M), 3.0, device)
    n_hot = int(round(0.05 * rows))
    hot = torch.randperm(rows, generator=g, device=device)[:n_hot]
    col = torch.randint(2 * hc, M, (n_hot,), generator=g, device=device)
    logits[hot, col] += 40.0
    scale = torch.ones(3, dtype=torch.float32, device=device)
    base = torch.zeros(M, dtype=torch.float32, device=device)
    return dict(mixes=logits, scale=scale, base=base, hot_rows=hot, hot_cols=col)


def long_prefill(seed: int = 0, device="cpu", layers: int = 40, pool: int = 4, w: Workload = LONG_PREFILL):
    """B=2, T=32768, d=5120, bf16 streams: independent (attention, FFN) mix
    parameters for each of ``layers`` layers (scale ~ U(0.5, 2)), streams
    x [n, 4, d] ~ N(0, 1), a pool of ``pool`` sublayer outputs [n, d] ~ N(0, 1)
    that the chain's sublayers cycle through (sublayer k uses pool[k % pool]),
    and the previous call whose pre weights collapse the first sublayer.

    Draw order: layer parameters (attention, FFN per layer), streams, pool,
    previous call. Sized for generation on the GPU (the fp32 draw of the streams
    alone is 5.4 GB)."""
    g = generator(seed, device)
    params = [(mix_params(g, w.hc, w.d, "uniform", device), mix_params(g, w.hc, w.d, "uniform", device))
              for _ in range(layers)]
    x = streams(g, w.n, w.hc, w.d, w.dtype, device=device)
    f_pool = [sublayer_output(g, w.n, w.d, w.dtype, device) for _ in range(pool)]
    prev = previous_call(g, w.n, w.hc, device)
    return dict(workload=w, params=params, x=x, f_pool=f_pool, prev=prev)
