"""Comparison rule shared by the GPU parity tests (not a test module).

An element passes when |got - ref| <= tol * max(|ref|, rho), where rho guards values
that cancel to near zero: the RMS of the reference token's row for streams, the
collapsed input and the mixes; 1 for the coefficients pre, post and comb, which are
O(1) by construction (comb entries lie in [0, 1] and its columns sum to one).

Tolerances: 1e-5 for fp32 results computed from exact inputs, 2e-2 for results of
bf16 stream configurations (the bf16 spacing is 2^-8 relative, so one rounding
difference is far inside it).
"""
import os
import sys

import torch

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def max_rel_err(got: torch.Tensor, ref: torch.Tensor, rho="row", tokens_dims=1) -> float:
    g = got.detach().to("cpu", torch.float64)
    r = ref.detach().to("cpu", torch.float64)
    assert g.shape == r.shape, (tuple(g.shape), tuple(r.shape))
    if g.numel() == 0:
        return 0.0
    if not torch.isfinite(g).all():
        return float("inf")
    lead = 1
    for s in r.shape[:tokens_dims]:
        lead *= s
    g2, r2 = g.reshape(lead, -1), r.reshape(lead, -1)
    if rho == "row":
        rho_t = r2.pow(2).mean(1, keepdim=True).sqrt()
    else:
        rho_t = torch.full((lead, 1), float(rho), dtype=torch.float64)
    den = torch.maximum(r2.abs(), rho_t)
    diff = (g2 - r2).abs()
    # an all-zero reference row (den == 0) must be matched exactly
    ratio = torch.where(den > 0, diff / den.clamp_min(1e-300),
                        torch.where(diff > 0, torch.full_like(diff, float("inf")), torch.zeros_like(diff)))
    return ratio.max().item()


def record(name: str, err: float, tol: float, gate: bool = True) -> float:
    """Prints a comparison's worst error, appends it to the margin log named by the
    HC_PARITY_LOG environment variable (test id, name, error, tolerance, "gate" or
    "report"; tab separated), and asserts it is within the tolerance (unless gate is
    False: a figure that is reported, not held to the tolerance)."""
    print(f"  {name:<28s} max rel err {err:.3e} (tol {tol:g})", flush=True)
    sys.stdout.flush()
    log = os.environ.get("HC_PARITY_LOG")
    if log:
        test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
        with open(log, "a") as fh:
            fh.write(f"{test}\t{name}\t{err:.6e}\t{tol:g}\t{'gate' if gate else 'report'}\n")
    assert err <= tol or not gate, f"{name}: max relative error {err:.3e} > {tol:g}"
    return err


def check(name: str, got, ref, tol: float, rho="row", tokens_dims=1) -> float:
    return record(name, max_rel_err(got, ref, rho, tokens_dims), tol)


def rho_for(key: str):
    k = key.lower()
    if k.startswith(("pre", "post", "comb")) or k.endswith(("pre", "post", "comb")):
        return 1.0
    return "row"
