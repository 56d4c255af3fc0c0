"""The binding refuses tensors whose sizes do not match the call before anything is
launched: the library reads and writes exactly the element counts the shapes imply,
so a short buffer would otherwise be read or written past its end on the GPU."""
import pytest
import torch

import hyper_connection_residual_mixes_amd as hc

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
N, D = 8, 64


def _z(*shape, dtype=torch.float32):
    return torch.zeros(*shape, dtype=dtype, device=DEV)


def test_post_short_sublayer_output():
    with pytest.raises(ValueError, match="f must hold"):
        hc.hc_post(_z(N * D - 8), _z(N, 4, D), _z(N, 4), _z(N, 4, 4))


def test_post_short_comb_and_out():
    with pytest.raises(ValueError, match="comb must hold"):
        hc.hc_post(_z(N, D), _z(N, 4, D), _z(N, 4), _z(N, 4))
    with pytest.raises(ValueError, match="out must hold"):
        hc.hc_post(_z(N, D), _z(N, 4, D), _z(N, 4), _z(N, 4, 4), out=_z(N, 2, D))


def test_pre_short_weights_and_output():
    with pytest.raises(ValueError, match="pre_mix must hold"):
        hc.hc_pre(_z(N, 4, D), _z(N, 3))
    with pytest.raises(ValueError, match="y must hold"):
        hc.hc_pre(_z(N, 4, D), _z(N, 4), out=_z(N, D // 2))


def test_mixes_wrong_projection_size():
    with pytest.raises(ValueError, match="hc_fn must hold"):
        hc.hc_mixes(_z(N, 4, D), _z(24, 4 * D - 1))


def test_split_short_parameters():
    with pytest.raises(ValueError, match="hc_scale must hold"):
        hc.hc_split_sinkhorn(_z(N, 24), _z(2), _z(24))
    with pytest.raises(ValueError, match="hc_base must hold"):
        hc.hc_split_sinkhorn(_z(N, 24), _z(3), _z(23))
    with pytest.raises(ValueError, match="comb must hold"):
        hc.hc_split_sinkhorn(_z(N, 24), _z(3), _z(24), out=(_z(N, 4), _z(N, 4), _z(N, 4)))


def test_fused_step_short_inputs():
    x, fn, s, b = _z(N, 4, D), _z(24, 4 * D), _z(3), _z(24)
    with pytest.raises(ValueError, match="hc_fn must hold"):
        hc.hc_fused_step(x, _z(24, D), s, b, pre_mix=_z(N, 4))
    with pytest.raises(ValueError, match="pre_mix must hold"):
        hc.hc_fused_step(x, fn, s, b, pre_mix=_z(N))
    with pytest.raises(ValueError, match="comb_prev must hold"):
        hc.hc_fused_step(x, fn, s, b, pre_mix=_z(N, 4), f_prev=_z(N, D), post_prev=_z(N, 4), comb_prev=_z(N, 4))
    with pytest.raises(ValueError, match="f_prev must hold"):
        hc.hc_fused_step(x, fn, s, b, pre_mix=_z(N, 4), f_prev=_z(N - 1, D), post_prev=_z(N, 4),
                         comb_prev=_z(N, 4, 4))


def test_rmsnorm_short_gain_and_scales():
    x = _z(N, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="gain must hold"):
        hc.rmsnorm_mxfp8(x, _z(D - 1))
    with pytest.raises(ValueError, match="scale must hold"):
        hc.rmsnorm_mxfp8(x, _z(D), scale=torch.zeros(N, 1, dtype=torch.uint8, device=DEV))


def test_well_formed_call_still_runs():
    y = hc.hc_pre(_z(N, 4, D), torch.full((N, 4), 0.25, device=DEV))
    torch.cuda.synchronize()
    assert y.shape == (N, D) and float(y.abs().max()) == 0.0
