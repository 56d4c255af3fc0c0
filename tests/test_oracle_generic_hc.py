"""Pins of the oracle for stream counts other than four (no GPU).

The "Stream combination" page's split kernel and the "Block" page are written for
any stream count hc (the released configuration uses 4) and any number of Sinkhorn
rounds: the mix numbers of a token are laid out as [pre (hc) | post (hc) | comb
(hc x hc, row-major)], (2 + hc) * hc in all, and the projection reads the hc
streams flattened in (stream, channel) order. These pins fix that layout and the
arithmetic for hc = 1, 2, 3, 5, 8 with hand-worked cases and closed forms.
"""
import math

import pytest
import torch

import oracle

EPS = 1e-6
HCS = [1, 2, 3, 5, 8]


def _f32(v: float) -> float:
    return float(torch.tensor(v, dtype=torch.float32))


def _m(hc):
    return (2 + hc) * hc


@pytest.mark.parametrize("hc", HCS)
@pytest.mark.parametrize("iters", [1, 3, 20])
def test_uniform_comb_closed_form(hc, iters):
    """All logits and offsets 0: pre = sigmoid(0) + eps, post = 1, and the comb stays
    uniform. Its value follows one normalisation of a constant hc x hc matrix,
    v <- v / (hc v + eps), applied once after the softmax (the first column step)
    and twice per later round, from v0 = 1/hc + eps. eps = 0.1 makes every eps term
    visible; a divisor of 4 instead of hc, or a wrong round count, fails."""
    eps = 0.1
    pre, post, comb = oracle.hc_split_sinkhorn(torch.zeros(1, _m(hc)), torch.ones(3), torch.zeros(_m(hc)),
                                               hc_mult=hc, sinkhorn_iters=iters, eps=eps)
    assert torch.equal(pre, torch.full((1, hc), _f32(0.5 + eps)))
    assert torch.equal(post, torch.ones(1, hc))
    v = 1.0 / hc + eps
    for _ in range(1 + 2 * (iters - 1)):
        v = v / (hc * v + eps)
    assert torch.allclose(comb, torch.full((1, hc, hc), _f32(v)), rtol=2e-7, atol=0)


@pytest.mark.parametrize("hc", [2, 3, 5, 8])
def test_cyclic_permutation_pins_comb_layout(hc):
    """Comb logits sit at mixes[2 hc + j hc + k]. A cyclic pattern L[j][(j+1) % hc] = 30
    gives, after the softmax + eps, equal row and column sums, so every normalisation
    scales all entries by 1/(S + eps) for the current common sum S: the final entries
    are (p + eps) * prod and (q + eps) * prod. A transposed or shifted layout fails."""
    Lbig = 30.0
    m = torch.zeros(1, _m(hc))
    for j in range(hc):
        m[0, 2 * hc + j * hc + (j + 1) % hc] = Lbig
    _, _, comb = oracle.hc_split_sinkhorn(m, torch.ones(3), torch.zeros(_m(hc)), hc_mult=hc)
    e = math.exp(-Lbig)
    p, q = 1 / (1 + (hc - 1) * e), e / (1 + (hc - 1) * e)
    S, fac = p + (hc - 1) * q + hc * EPS, 1.0
    for _ in range(1 + 2 * 19):
        fac /= S + EPS
        S = S / (S + EPS)
    for j in range(hc):
        for k in range(hc):
            want = (p + EPS) * fac if k == (j + 1) % hc else (q + EPS) * fac
            assert comb[0, j, k].item() == pytest.approx(want, rel=1e-6, abs=1e-12), (j, k)


@pytest.mark.parametrize("R", [1, 2, 5, 20])
def test_two_stream_triangular_closed_form(R):
    """hc = 2, eps = 0, logits 0 on [[1, 1], [0, 1]] and -1000 below the diagonal (its
    exponential underflows to 0). Row-then-column normalisation keeps the form
    [[1, x], [0, 1 - x]] after each column step with 1/x_R = 2R + 1, so after R
    rounds comb = [[1, 1/(2R+1)], [0, 2R/(2R+1)]]."""
    m = torch.zeros(1, 8)
    m[0, 4 + 2 * 1 + 0] = -1000.0
    _, _, comb = oracle.hc_split_sinkhorn(m, torch.ones(3), torch.zeros(8), hc_mult=2, sinkhorn_iters=R,
                                          eps=0.0)
    c = comb[0]
    assert c[0, 0].item() == 1.0 and c[1, 0].item() == 0.0
    assert c[0, 1].item() == _f32(1 / (2 * R + 1))
    assert c[1, 1].item() == _f32(2 * R / (2 * R + 1))


@pytest.mark.parametrize("hc", [1, 3, 8])
def test_split_pre_post_index_ranges(hc):
    """pre[j] = sigmoid(s0 m[j] + b[j]) + eps and post[j] = 2 sigmoid(s1 m[hc + j] + b[hc + j]):
    m[j] = ln(a_j) / s0 gives sigmoid(ln a) = a / (1 + a); the post logits count down."""
    a = [1.0 + 0.5 * j for j in range(hc)]
    m = torch.zeros(1, _m(hc))
    for j in range(hc):
        m[0, j] = math.log(a[j]) / 2.0
        m[0, hc + j] = math.log(a[hc - 1 - j])
    pre, post, _ = oracle.hc_split_sinkhorn(m, torch.tensor([2.0, 1.0, 1.0]), torch.zeros(_m(hc)), hc_mult=hc)
    for j in range(hc):
        assert pre[0, j].item() == pytest.approx(a[j] / (1 + a[j]) + EPS, rel=1e-7)
        assert post[0, j].item() == pytest.approx(2 * a[hc - 1 - j] / (1 + a[hc - 1 - j]), rel=1e-7)


@pytest.mark.parametrize("hc", [1, 2, 3, 8])
def test_mixes_flatten_order_and_joint_rms(hc):
    """hc_mixes flattens the hc streams in (stream, channel) order and takes one RMS
    statistic over all hc * d entries. x[j][e] = +-2 (so r = 1/2); one-hot row i picks
    flat index c_i = j d + e, giving m_i = x_flat[c_i] / 2; an all-ones row gives
    r * sum(x)."""
    d = 4
    g = torch.Generator().manual_seed(hc)
    sign = torch.where(torch.rand(hc * d, generator=g) < 0.5, -1.0, 1.0)
    x = (2.0 * sign).reshape(1, hc, d)
    M = _m(hc)
    W = torch.zeros(M, hc * d)
    idx = [(7 * i + 3) % (hc * d) for i in range(M - 1)]
    for i, c in enumerate(idx):
        W[i, c] = 1.0
    W[M - 1] = 1.0
    m = oracle.hc_mixes(x, W)
    for i, c in enumerate(idx):
        assert m[0, i].item() == sign[c].item(), (i, c)
    assert m[0, M - 1].item() == pytest.approx(0.5 * 2.0 * sign.sum().item(), abs=1e-6)


@pytest.mark.parametrize("hc", [1, 3, 8])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pre_one_hot_selects_stream(hc, dtype):
    """hc_pre: y = sum_j pre_mix[j] x[j]; a one-hot pre_mix returns that stream exactly."""
    g = torch.Generator().manual_seed(1)
    x = torch.randn(3, hc, 40, generator=g).to(dtype)
    for j in range(hc):
        pm = torch.zeros(3, hc)
        pm[:, j] = 1.0
        assert torch.equal(oracle.hc_pre(x, pm), x[:, j])


@pytest.mark.parametrize("hc", [2, 3, 8])
def test_post_permutation_and_orientation(hc):
    """hc_post: new stream k = post[k] f + sum_j comb[j][k] res[j]. A permutation comb
    (old j -> new perm[j]) with post = 0 moves the streams; comb = I with post = 1 adds
    f to every stream."""
    res = torch.arange(2 * hc * 8, dtype=torch.float32).reshape(2, hc, 8)
    f = torch.full((2, 8), 1000.0)
    out = oracle.hc_post(f, res, torch.ones(2, hc), torch.eye(hc).expand(2, hc, hc))
    assert torch.equal(out, res + 1000.0)
    perm = [(3 * j + 1) % hc for j in range(hc)] if hc != 3 else [2, 0, 1]
    assert sorted(perm) == list(range(hc))
    P = torch.zeros(hc, hc)
    for j, k in enumerate(perm):
        P[j, k] = 1.0
    out = oracle.hc_post(f, res, torch.zeros(2, hc), P.expand(2, hc, hc))
    for j, k in enumerate(perm):
        assert torch.equal(out[:, k], res[:, j])
