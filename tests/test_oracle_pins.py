"""Pins of the CPU oracle against facts the pages and mathematics fix (no GPU).

Each test names the passage it pins. None of them re-types the oracle's general
algorithm: they use hand-worked cases, closed forms of special cases, invariants
the pages state, and library routines for the rounding rule.
"""
import json
import math
import os

import pytest
import torch

import hc_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = 1e-6


def _f32(v: float) -> float:
    return float(torch.tensor(v, dtype=torch.float32))


# ----------------------------------------------------------------- parameters
def test_page_parameter_counts():
    """"Stream combination" page (summary, parameter table) and "Block" page
    (parameter table): 24 = (2+4)*4 mix numbers, 17 comb parameters per instance
    (85 over 5 layers), 491,547 parameters per stream-weight instance at d=5120."""
    g = json.load(open(os.path.join(GOLDEN, "page_figures.json")))
    hc, d = g["stream_weight_instance_parameters"]["hc"], g["stream_weight_instance_parameters"]["d"]
    shapes = oracle.param_shapes(hc, d)
    assert shapes["hc_fn"][0] == g["mix_numbers_per_token"]["value"]
    total = sum(math.prod(s) for s in shapes.values())
    assert total == g["stream_weight_instance_parameters"]["value"]
    offs, scales = oracle.comb_param_indices(hc)
    assert len(offs) == g["comb_component_parameters"]["offsets"]
    assert len(offs) + len(scales) == g["comb_component_parameters"]["value"]
    assert 5 * (len(offs) + len(scales)) == g["comb_component_parameters_5_layers"]["value"]
    cfg = g["released_config"]
    assert (oracle.HC_MULT, oracle.SINKHORN_ITERS, oracle.HC_EPS, oracle.NORM_EPS) == (
        cfg["hc_mult"], cfg["hc_sinkhorn_iters"], cfg["hc_eps"], cfg["norm_eps"])


# ------------------------------------------------------------ bf16 rounding
def test_bf16_rounding_ties_to_even():
    """Diagram block "Cast" (FP32 -> BF16: nearest representable number); ties to even."""
    one = 0x3F80
    assert oracle.round_bf16_bits(1.0 + 2.0**-8) == one            # tie -> even (down)
    assert oracle.round_bf16_bits(1.0 + 3 * 2.0**-8) == one + 2    # tie -> even (up)
    assert oracle.round_bf16_bits(1.0 + 2.0**-8 + 2.0**-30) == one + 1
    assert oracle.round_bf16_bits(-(1.0 + 2.0**-8)) == 0xBF80
    assert oracle.round_bf16_bits(0.0) == 0


def test_bf16_rounding_subnormal_range():
    """Below 2^-126 bf16 keeps the fp32 subnormal grid, multiples of 2^-133 (Diagram
    block "Cast": nearest representable number; ties to even). Hand-worked values:
    the grid point itself, ties on both sides of an even unit, the tie at half a unit
    (to zero), and the largest subnormal rounding up into the smallest normal."""
    u = 2.0**-133
    assert oracle.round_bf16_bits(u) == 0x0001
    assert oracle.round_bf16_bits(1.5 * u) == 0x0002      # tie 1 | 2 -> 2 (even)
    assert oracle.round_bf16_bits(2.5 * u) == 0x0002      # tie 2 | 3 -> 2 (even)
    assert oracle.round_bf16_bits(0.5 * u) == 0x0000      # tie 0 | 1 -> 0 (even)
    assert oracle.round_bf16_bits(0.5000001 * u) == 0x0001
    assert oracle.round_bf16_bits(-3.0 * u) == 0x8003
    assert oracle.round_bf16_bits(126.5 * u) == 0x007E    # tie 126 | 127 -> 126
    assert oracle.round_bf16_bits(127.5 * u) == 0x0080    # tie 127 | 128 -> 2^-126 (normal)
    assert oracle.round_bf16_bits(2.0**-126 - 2.0**-136) == 0x0080
    assert oracle.round_bf16_bits(1e-45) == 0x0000        # far below half a unit


def test_bf16_rounding_overflow_range():
    """Top of the range: the largest finite bf16 is (2 - 2^-7) * 2^127 (0x7F7F); the
    midpoint to 2^128 rounds to the even neighbour, which is infinity; beyond it
    everything is infinity with the sign kept."""
    top = (2.0 - 2.0**-7) * 2.0**127
    assert oracle.round_bf16_bits(top) == 0x7F7F
    assert oracle.round_bf16_bits((2.0 - 2.0**-8 - 2.0**-20) * 2.0**127) == 0x7F7F
    assert oracle.round_bf16_bits((2.0 - 2.0**-8) * 2.0**127) == 0x7F80   # tie -> even (inf)
    assert oracle.round_bf16_bits(2.0**128) == 0x7F80
    assert oracle.round_bf16_bits(1e39) == 0x7F80
    assert oracle.round_bf16_bits(-1e300) == 0xFF80
    assert oracle.round_bf16_bits(-top) == 0xFF7F


def test_bf16_rounding_matches_torch_on_fp32_values():
    """Library routine: torch's fp32 -> bf16 conversion is round-to-nearest-even; on
    fp32-representable inputs the oracle's direct fp64 -> bf16 rounding must agree."""
    g = torch.Generator().manual_seed(3)
    v = torch.randn(4000, generator=g) * torch.exp(torch.randn(4000, generator=g) * 8)
    want = v.to(torch.bfloat16).view(torch.int16).to(torch.int32) & 0xFFFF
    got = torch.tensor([oracle.round_bf16_bits(float(a)) for a in v], dtype=torch.int32)
    assert torch.equal(got, want)


# ---------------------------------------------------------------- hc_mixes
def _onehot_rows(hc, d, idx):
    M = (2 + hc) * hc
    W = torch.zeros(M, hc * d)
    for i, c in enumerate(idx):
        W[i, c] = 1.0
    return W


def test_mixes_hand_case_d4_flatten_order_and_joint_rms():
    """"Block" page, hc_mixes: the 4 streams are flattened in (stream, channel) order,
    ONE RMS statistic is taken over all 4*d entries, and the projection is scaled by it.
    Hand case d=4: stream 0 = [4,4,4,4], others 0 -> mean(x^2) = 64/16 = 4, r = 1/2."""
    hc, d = 4, 4
    x = torch.zeros(1, hc, d)
    x[0, 0] = 4.0
    x[0, 1, 0] = 0.0
    # one-hot at flat index 1 = (stream 0, channel 1) and at 4 = (stream 1, channel 0)
    idx = [1, 4, 0, 3] + [5] * 20
    W = _onehot_rows(hc, d, idx)
    W[23] = 1.0                          # all-ones row: r * sum(x) = 0.5 * 16 = 8
    m = oracle.hc_mixes(x, W)
    assert m[0, 0].item() == 2.0         # 0.5 * x[0][1]
    assert m[0, 1].item() == 0.0         # 0.5 * x[1][0]
    assert m[0, 2].item() == 2.0
    assert m[0, 23].item() == 8.0


def test_mixes_hand_case_distinct_values():
    """Same passage; distinct entries pin the flat index c = j*d + e exactly.
    x[j][e] = +-2 (so r = 1/2), one-hot row i picks flat index c_i -> m_i = x_flat[c_i] / 2."""
    hc, d = 4, 4
    sign = torch.tensor([1, -1, -1, 1, 1, 1, -1, -1, -1, 1, 1, -1, 1, -1, 1, 1], dtype=torch.float32)
    x = (2.0 * sign).reshape(1, hc, d)
    idx = list(range(16)) + [15, 14, 13, 12, 1, 2, 3, 4]
    m = oracle.hc_mixes(x, _onehot_rows(hc, d, idx))
    want = torch.tensor([sign[c].item() for c in idx])
    assert torch.equal(m[0], want)


def test_mixes_scale_invariance():
    """The mixes see the streams only through x * rsqrt(mean(x^2)), so scaling a token's
    streams by a > 0 leaves them unchanged (up to the 1e-20 epsilon and rounding).
    This is what keeps the x50 outlier tokens of the prefill workload ordinary."""
    g = torch.Generator().manual_seed(0)
    hc, d = 4, 64
    x = torch.randn(3, hc, d, generator=g)
    W = torch.randn(24, hc * d, generator=g) / math.sqrt(hc * d)
    m1 = oracle.hc_mixes(x, W)
    m2 = oracle.hc_mixes(x * 50.0, W)
    assert torch.allclose(m1, m2, rtol=1e-6, atol=1e-7)
    xb = x.to(torch.bfloat16)
    assert torch.equal(oracle.hc_mixes(xb, W), oracle.hc_mixes(xb * 64, W))  # exact power of 2


def test_mixes_norm_eps_is_1e_minus_20():
    """Released configuration: norm_eps = 1e-20 (not hc_eps). Tiny streams of 1e-12:
    mean(x^2) = 1e-24, r = 1/sqrt(1e-24 + 1e-20); all-ones row -> 16e-12 * r."""
    hc, d = 4, 4
    x = torch.full((1, hc, d), 1e-12, dtype=torch.float32)
    xv = float(x[0, 0, 0])
    W = torch.ones(24, 16)
    m = oracle.hc_mixes(x, W)
    want = 16 * xv / math.sqrt(xv * xv + 1e-20)
    assert m[0, 0].item() == pytest.approx(want, rel=1e-6)
    z = oracle.hc_mixes(torch.zeros(2, hc, d), W)
    assert torch.equal(z, torch.zeros_like(z))


# ------------------------------------------------------------ split / Sinkhorn
def _logits(hc=4):
    return torch.zeros(1, (2 + hc) * hc)


@pytest.mark.parametrize("eps", [EPS, 0.1, 0.5])
def test_split_sigmoid_zero_and_uniform_comb_closed_form(eps):
    """"Stream combination" code section and diagram blocks sigma / 2 sigma / x+eps:
    with all logits and offsets 0, pre = sigmoid(0) + eps, post = 2 sigmoid(0) = 1,
    and the uniform comb stays uniform; its value follows the scalar recurrence of
    one normalisation of a constant 4x4 matrix, v <- v / (4v + eps), applied
    1 (first column step) + 2*19 times to v0 = 1/4 + eps. At the released eps the
    recurrence sits at its fixed point; the larger eps values make every one of the
    39 eps terms (and the one after the softmax) visible in fp32."""
    pre, post, comb = oracle.hc_split_sinkhorn(_logits(), torch.ones(3), torch.zeros(24), eps=eps)
    assert torch.equal(pre, torch.full((1, 4), _f32(0.5 + eps)))
    assert torch.equal(post, torch.ones(1, 4))
    v = 0.25 + eps
    for _ in range(1 + 2 * 19):
        v = v / (4 * v + eps)
    assert comb[0, 0, 0].item() == _f32(v)
    assert torch.equal(comb, torch.full((1, 4, 4), comb[0, 0, 0].item()))


def test_split_sigmoid_hand_values_and_scale_indices():
    """pre[j] = sigmoid(s0*m[j] + b[j]) + eps, post[j] = 2 sigmoid(s1*m[4+j] + b[4+j]).
    With s = (2, 1, 0.5): m[j] = ln(a_j)/2 gives sigmoid(ln a) = a/(1+a)."""
    a = [1.0, 3.0, 1 / 3, 7.0]
    m = torch.zeros(1, 24)
    for j in range(4):
        m[0, j] = math.log(a[j]) / 2          # scaled by s0 = 2
        m[0, 4 + j] = math.log(a[3 - j])      # scaled by s1 = 1
    base = torch.zeros(24)
    s = torch.tensor([2.0, 1.0, 0.5])
    pre, post, _ = oracle.hc_split_sinkhorn(m, s, base)
    for j in range(4):
        assert pre[0, j].item() == pytest.approx(a[j] / (1 + a[j]) + EPS, rel=1e-7)
        assert post[0, j].item() == pytest.approx(2 * a[3 - j] / (1 + a[3 - j]), rel=1e-7)
    # the same numbers through the offsets instead of the logits
    base2 = torch.zeros(24)
    for j in range(4):
        base2[j] = math.log(a[j])
        base2[4 + j] = math.log(a[3 - j])
    pre2, post2, _ = oracle.hc_split_sinkhorn(torch.zeros(1, 24), s, base2)
    assert torch.allclose(pre2, pre, rtol=1e-7) and torch.allclose(post2, post, rtol=1e-7)


def test_sinkhorn_cyclic_permutation_closed_form_pins_layout_and_eps():
    """Comb logits are stored row-major at mixes[8 + 4j + k] ("Stream combination" code).
    A cyclic pattern L[j][(j+1)%4] = 30 gives, after the row softmax + eps, a matrix
    whose row and column sums are all equal, so every normalisation multiplies all
    entries by the same factor 1/(S+eps) with S the current common sum. Final
    entries are then (p+eps)*prod and (q+eps)*prod. Pins the comb index layout, the
    orientation, and the +eps added after the softmax (off-pattern entries ~ eps)."""
    Lbig = 30.0
    m = torch.zeros(1, 24)
    for j in range(4):
        m[0, 8 + 4 * j + (j + 1) % 4] = Lbig
    _, _, comb = oracle.hc_split_sinkhorn(m, torch.ones(3), torch.zeros(24))
    e = math.exp(-Lbig)
    p, q = 1 / (1 + 3 * e), e / (1 + 3 * e)
    S, fac = p + 3 * q + 4 * EPS, 1.0
    for _ in range(1 + 2 * 19):
        fac /= S + EPS
        S = S / (S + EPS)
    for j in range(4):
        for k in range(4):
            want = (p + EPS) * fac if k == (j + 1) % 4 else (q + EPS) * fac
            assert comb[0, j, k].item() == _f32(want), (j, k)
    assert comb[0, 0, 1] > 0.99 and comb[0, 1, 0] < 2e-6   # not the transpose


def test_sinkhorn_triangular_block_closed_form_pins_rounds_and_order():
    """Slowly converging case with an exact answer (eps = 0). Logits 0 on the block
    pattern [[1,1],[0,1]] (x) ones(2,2) and -1000 elsewhere (exp underflows to 0).
    The 4x4 iterates are (2x2 iterate) (x) ones(2,2)/2, and for the 2x2 matrix
    [[1,1],[0,1]] row-then-column normalisation keeps the form [[1, x],[0, 1-x]]
    after each column step with 1/x_r = 2r + 1 (x_1 = 1/3 after the first round).
    Hence after R rounds: comb[0..1][2..3] = 1/(2(2R+1)), comb[2..3][2..3] = R/(2R+1).
    Pins: the number of rounds (R = sinkhorn_iters), row step before column step,
    and the column step last."""
    m = torch.full((1, 24), -1000.0)
    for j in range(4):
        for k in range(4):
            if not (j >= 2 and k < 2):
                m[0, 8 + 4 * j + k] = 0.0
    for R in (1, 2, 5, 20):
        _, _, comb = oracle.hc_split_sinkhorn(m, torch.ones(3), torch.zeros(24),
                                              sinkhorn_iters=R, eps=0.0)
        c = comb[0]
        for j in (0, 1):
            for k in (0, 1):
                assert c[j, k].item() == 0.5
                assert c[j, k + 2].item() == _f32(1 / (2 * (2 * R + 1))), (R, j, k)
                assert c[j + 2, k].item() == 0.0
                assert c[j + 2, k + 2].item() == _f32(R / (2 * R + 1)), (R, j, k)
        assert torch.allclose(c.sum(0), torch.ones(4), atol=1e-7)   # columns exact


def test_sinkhorn_max_subtracted_softmax_is_finite():
    """The row softmax subtracts the row maximum before exp ("Stream combination" code):
    logits of 1000 must not overflow."""
    m = torch.zeros(1, 24)
    m[0, 8:24] = torch.tensor([1000.0, 0, 0, 0] * 4)
    _, _, comb = oracle.hc_split_sinkhorn(m, torch.ones(3), torch.zeros(24))
    assert torch.isfinite(comb).all()


def test_sinkhorn_eps_keeps_underflowed_entries_positive():
    """Diagram "First Sinkhorn Round": an entry whose exponential underflows to zero is
    lifted above zero by the eps added after the softmax."""
    m = torch.zeros(1, 24)
    for j in range(4):
        m[0, 8 + 5 * j] = -1000.0            # the diagonal underflows to exactly 0
    _, _, comb = oracle.hc_split_sinkhorn(m, torch.ones(3), torch.zeros(24))
    assert (comb > 0).all()
    _, _, comb0 = oracle.hc_split_sinkhorn(m, torch.ones(3), torch.zeros(24), eps=0.0)
    assert (torch.diagonal(comb0[0]) == 0).all() and (comb0 > 0).sum() == 12


def test_split_invariants_on_stress_sample():
    """Diagram blocks sigma / 2 sigma / "Sinkhorn Round": pre in [eps, 1+eps], post in
    [0, 2], comb >= 0; the last step is a column normalisation, so every column sums
    to s/(s+eps) (within eps + fp32 rounding of 1); rows only sum to ABOUT one: for
    the wide N(0, 3) logits of the stress workload 20 rounds leave up to ~5% (the +40
    rows included), for unit-scale logits typically ~1e-6. Run on a stress sample."""
    st = hc_inputs.stress(seed=0, rows=4096)
    pre, post, comb = oracle.hc_split_sinkhorn(st["mixes"], st["scale"], st["base"])
    assert (pre >= _f32(EPS)).all() and (pre <= 1 + 2 * EPS).all()
    assert (post >= 0).all() and (post <= 2).all()
    assert (comb >= 0).all()
    col = comb.double().sum(1)
    assert (col - 1).abs().max().item() < 2.5e-6
    hot = torch.zeros(4096, dtype=torch.bool)
    hot[st["hot_rows"]] = True
    row = comb.double().sum(2)
    assert (row - 1).abs().max().item() < 0.1
    assert (row[~hot] - 1).abs().median().item() < 1e-3
    m = torch.randn(4096, 24, generator=torch.Generator().manual_seed(0))
    _, _, c1 = oracle.hc_split_sinkhorn(m, torch.ones(3), torch.zeros(24))
    assert ((c1.double().sum(2) - 1).abs().amax(1) < 1e-4).float().mean() > 0.999


def test_split_rejects_zero_rounds():
    with pytest.raises(ValueError):
        oracle.hc_split_sinkhorn(_logits(), torch.ones(3), torch.zeros(24), sinkhorn_iters=0)


# ------------------------------------------------------------------ hc_pre
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pre_one_hot_selects_stream(dtype):
    """"Block" page hc_pre: y = sum_j pre_mix[j] * x[j]; a one-hot pre_mix returns
    that stream exactly."""
    g = torch.Generator().manual_seed(1)
    x = torch.randn(3, 4, 40, generator=g).to(dtype)
    for j in range(4):
        pm = torch.zeros(3, 4)
        pm[:, j] = 1.0
        assert torch.equal(oracle.hc_pre(x, pm), x[:, j])


def test_pre_hand_case_and_linearity():
    """Hand case d=4: streams 1, 10, 100, 1000 times [1,2,3,4] and weights
    [1, 1/2, 1/4, 1/8] give 156 * [1,2,3,4]; doubling the weights doubles y."""
    base = torch.tensor([1.0, 2, 3, 4])
    x = torch.stack([base * s for s in (1, 10, 100, 1000)])[None]
    pm = torch.tensor([[1.0, 0.5, 0.25, 0.125]])
    y = oracle.hc_pre(x, pm)
    assert torch.equal(y, (156 * base)[None])
    assert torch.equal(oracle.hc_pre(x, 2 * pm), 2 * y)
    xb = x.to(torch.bfloat16)
    assert oracle.hc_pre(xb, pm).dtype == torch.bfloat16


# ----------------------------------------------------------------- hc_post
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_post_orientation_single_entry(dtype):
    """"Block" page hc_post: new stream k = post[k]*f + sum_j comb[j][k]*res[j]. A
    single 1 at comb[1][3] with post = 0 copies OLD stream 1 into NEW stream 3 and
    leaves the others zero (comb^T would copy 3 into 1)."""
    g = torch.Generator().manual_seed(2)
    res = torch.randn(2, 4, 24, generator=g).to(dtype)
    f = torch.randn(2, 24, generator=g).to(dtype)
    comb = torch.zeros(2, 4, 4)
    comb[:, 1, 3] = 1.0
    out = oracle.hc_post(f, res, torch.zeros(2, 4), comb)
    assert torch.equal(out[:, 3], res[:, 1])
    for k in (0, 1, 2):
        assert (out[:, k] == 0).all()


def test_post_identity_and_permutation():
    """comb = I, post = 1 gives f + res[k]; a permutation comb permutes the streams."""
    res = torch.arange(2 * 4 * 8, dtype=torch.float32).reshape(2, 4, 8)
    f = torch.full((2, 8), 1000.0)
    out = oracle.hc_post(f, res, torch.ones(2, 4), torch.eye(4).expand(2, 4, 4))
    assert torch.equal(out, res + 1000.0)
    perm = [2, 0, 3, 1]                           # old j -> new perm[j]
    P = torch.zeros(4, 4)
    for j, k in enumerate(perm):
        P[j, k] = 1.0
    out = oracle.hc_post(f, res, torch.zeros(2, 4), P.expand(2, 4, 4))
    for j, k in enumerate(perm):
        assert torch.equal(out[:, k], res[:, j])


def test_post_stream_sum_identity():
    """Diagram "Sinkhorn Round": with comb rows summing to one the sum of the streams
    is kept. In general sum_k out[k] = (sum_k post[k]) f + sum_j rowsum_j res[j]."""
    g = torch.Generator().manual_seed(4)
    n, d = 5, 32
    res = torch.randn(n, 4, d, generator=g)
    f = torch.randn(n, d, generator=g)
    post = torch.rand(n, 4, generator=g) * 2
    comb = torch.rand(n, 4, 4, generator=g)
    out = oracle.hc_post(f, res, post, comb).double()
    want = post.double().sum(1, keepdim=True) * f.double() + (
        comb.double().sum(2, keepdim=True) * res.double()).sum(1)
    assert torch.allclose(out.sum(1), want, rtol=0, atol=1e-5)


# ----------------------------------------------------- block wiring (Single-Pass mHC)
def test_block_wiring_collapse_uses_previous_sublayer_pre():
    """"Block" page forward and diagram "Single-Pass mHC": attention collapses with the
    pre weights handed over from the previous layer, the FFN collapses with the pre
    weights attention computed, and the FFN's own pre weights go to the next layer.
    Changing pre_mix therefore changes the attention collapse and nothing else."""
    inp = hc_inputs.tiny(seed=0)
    pi = torch.rand(16, 4, generator=torch.Generator().manual_seed(9))
    a = oracle.block(inp["x"], pi, inp["attn"], inp["ffn"],
                     inp["f_attn"], inp["f_ffn"])
    b = oracle.block(inp["x"], pi * 0.5, inp["attn"], inp["ffn"],
                     inp["f_attn"], inp["f_ffn"])
    for k in a:
        if k == "yA":
            assert not torch.equal(a[k], b[k])
        else:
            assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["yF"], oracle.hc_pre(a["x1"], a["preA"]))
    assert not torch.equal(a["yF"], oracle.hc_pre(a["x1"], a["preF"]))


# ------------------------------------------------ RMSNorm and MXFP8 cast (next rows)
def _group_with_unit_scale(vals):
    """Groups of 32 whose first element is 448, so the group scale is 2^0 and the
    codes of the other 31 elements are the plain E4M3 codes of their values."""
    vals = list(vals)
    rows = []
    for i in range(0, len(vals), 31):
        chunk = vals[i:i + 31]
        chunk += [0.0] * (31 - len(chunk))
        rows.append([448.0] + chunk)
    return torch.tensor(rows, dtype=torch.float32)


def test_e4m3_codes_match_torch_float8():
    """E4M3 rounding ([Diagram] "Cast to MXFP8": nearest E4M3 number) against
    torch's independent float8_e4m3fn conversion: random values over the whole
    range, the subnormal range, and exact midpoints between neighbouring codes."""
    g = hc_inputs.generator(3)
    vals = (torch.rand(3000, generator=g) * 2 - 1) * 448
    vals = torch.cat([vals, (torch.rand(1000, generator=g) * 2 - 1) * 2.0 ** -6])
    mids = []
    for e in range(-6, 8):
        for m in range(8):
            mids.append((1 + (m + 0.5) / 8) * 2.0 ** e)   # halfway between two codes
    for m in range(8):
        mids.append((m + 0.5) * 2.0 ** -9)                 # subnormal midpoints
    vals = torch.cat([vals, torch.tensor(mids), -torch.tensor(mids)])
    x = _group_with_unit_scale(vals.tolist())
    q, sc = oracle.mxfp8(x)
    assert (sc == 127).all()
    ref = x[:, 1:].to(torch.float8_e4m3fn).view(torch.uint8)
    assert torch.equal(q[:, 1:], ref)
    assert (q[:, 0] == 0x7E).all()                         # 448 is the largest finite code


def test_mxfp8_page_extremes_and_sign():
    """The page's statements: E4M3 tops out at 448 and flushes below 2^-9 without a
    scale; a value halfway to the smallest subnormal rounds to the even code 0;
    the sign of a value that rounds to zero is kept."""
    x = _group_with_unit_scale([2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -10, -2.0 ** -12, 447.0, -448.0])
    q, _ = oracle.mxfp8(x)
    assert q[0, 1:7].tolist() == [0x01, 0x00, 0x01, 0x80, 0x7E, 0xFE]


def test_mxfp8_group_scales_hand_cases():
    """UE8M0 scale = 2^ceil(log2(max(amax, 1e-4) / 448)), byte = exponent + 127."""
    cases = {   # amax -> exponent of the scale
        448.0: 0, 450.0: 1, 224.0: -1, 225.0: 0, 896.0: 1, 897.0: 2, 1.0: -8,
        1e-4: -22, 1e-6: -22, 0.0: -22, 3.5: -7, 3.0 * 2 ** 100: 93,   # 100 + log2(3/448) = 92.8
    }
    rows = [[a] + [0.0] * 31 for a in cases]
    q, sc = oracle.mxfp8(torch.tensor(rows, dtype=torch.float32))
    assert sc[:, 0].tolist() == [k + 127 for k in cases.values()]
    # 450 / 2 = 225 = 1.7578 * 2^7 -> mantissa 6.06 -> 6: code (7 + 7) << 3 | 6
    assert q[1, 0].item() == 0x76
    # a group whose amax is exactly 448 * 2^k is scaled to exactly 448
    q2, sc2 = oracle.mxfp8(torch.tensor([[448.0 * 8] + [-3.0] * 31], dtype=torch.float32))
    assert sc2.item() == 130 and q2[0, 0].item() == 0x7E
    # dequantised values stay within half an E4M3 step of the scaled input
    g = hc_inputs.generator(4)
    x = torch.randn(64, 256, generator=g) * torch.logspace(-6, 6, 64).unsqueeze(1)
    q3, sc3 = oracle.mxfp8(x)
    deq = q3.view(torch.float8_e4m3fn).float() * torch.pow(2.0, sc3.float() - 127).repeat_interleave(32, 1)
    s = torch.pow(2.0, sc3.float() - 127).repeat_interleave(32, 1)
    step = torch.where(x.abs() / s < 2 ** -6, torch.full_like(x, 2.0 ** -9), 2.0 ** (torch.floor(torch.log2((x.abs() / s).clamp_min(2 ** -6))) - 3))
    assert ((deq - x).abs() <= step * s / 2 * (1 + 1e-6)).all()


def test_rmsnorm_closed_forms():
    """RMSNorm ([Donor] RMSNorm passages; [Block] RMSNorm(dim, norm_eps)): a constant
    row maps to the gain (times its sign); (3, 4, 0, 0) has RMS 2.5 and maps to
    (1.2, 1.6, 0, 0) x gain; scaling a row by a power of two changes nothing; the
    epsilon keeps an all-zero row at zero."""
    gain = torch.tensor([0.5, 2.0, -1.0, 3.0])
    x = torch.tensor([[7.0, 7.0, 7.0, 7.0], [-0.25, -0.25, -0.25, -0.25], [3.0, 4.0, 0.0, 0.0],
                      [0.0, 0.0, 0.0, 0.0]])
    out = oracle.rmsnorm(x, gain)
    assert torch.allclose(out[0], gain, rtol=1e-7, atol=0)
    assert torch.allclose(out[1], -gain, rtol=1e-7, atol=0)
    assert torch.allclose(out[2], torch.tensor([0.6, 3.2, 0.0, 0.0]), rtol=1e-6, atol=0)
    assert torch.equal(out[3], torch.zeros(4))
    g = hc_inputs.generator(5)
    xr = torch.randn(8, 512, generator=g).to(torch.bfloat16)
    gr = torch.rand(512, generator=g) + 0.5
    assert torch.equal(oracle.rmsnorm(xr, gr), oracle.rmsnorm(xr * 8, gr))
    assert oracle.rmsnorm(xr, gr).dtype == torch.bfloat16


def test_rmsnorm_uses_norm_eps():
    """With eps = norm_eps = 1e-20 a tiny constant row still normalises to the gain;
    with a large eps the output shrinks by sqrt(ms / (ms + eps))."""
    x = torch.full((1, 64), 1e-6)
    gain = torch.ones(64)
    assert torch.allclose(oracle.rmsnorm(x, gain), torch.ones(1, 64), rtol=1e-6, atol=0)
    out = oracle.rmsnorm(torch.full((1, 64), 2.0), gain, norm_eps=12.0)   # 2 / sqrt(4 + 12)
    assert torch.allclose(out, torch.full((1, 64), 0.5), rtol=1e-7, atol=0)
