"""GPU AQN RMSNorm (qerl_aqn_rmsnorm) against the fp64 oracle: FP32 output
within 1e-5 relative per element, BF16 output the nearest-even rounding of
the exact value (one BF16 ulp allowed where the FP32 result sits on the other
side of a rounding boundary), noisy weight within 1e-6 relative."""
import numpy as np
import pytest
import torch

import oracle
import nvfp4_weight_only_quantize_amd as q
from nvfp4_weight_only_quantize_amd import synth
from parity import AQN_REL, bits_to_gpu, dev, gpu_bits

pytestmark = pytest.mark.gpu

SIGMA0, SIGMA1, STAGES, EPS = 1e-2, 5e-4, 10, 1e-6


def _run(m, h, sigma, seed, step, layer, x_seed, ldx_pad=0):
    x = synth.bf16_bits(synth.activation_bf16(m, h, seed=x_seed, outlier_col_frac=0.005))
    w = synth.norm_weight_f32(h, seed=x_seed + 1)
    xg = bits_to_gpu(x)
    if ldx_pad:
        xw = torch.zeros((m, h + ldx_pad), dtype=torch.bfloat16, device=dev())
        xw[:, :h] = xg
        xg = xw[:, :h]
    wn = torch.empty(h, dtype=torch.float32, device=dev())
    yf, yb = q.aqn_rmsnorm(xg, w.to(dev()), EPS, sigma, seed, step, layer, want_f32=True,
                           want_bf16=True, noisy_weight_out=wn)
    torch.cuda.synchronize()
    ref, wref = oracle.aqn_rmsnorm(x, w.numpy(), EPS, float(np.float32(sigma)), seed, step, layer)
    return yf.cpu().numpy().astype(np.float64), gpu_bits(yb), wn.cpu().numpy(), ref, wref


def _check(yf, yb_bits, wn, ref, wref, what=""):
    nz = ref != 0
    rel = np.abs(yf[nz] - ref[nz]) / np.abs(ref[nz])
    assert rel.max() <= AQN_REL, f"{what}: max rel {rel.max():.3e}"
    assert np.all(yf[~nz] == 0)
    np.testing.assert_allclose(wn, wref, rtol=1e-6, atol=0)
    # BF16 output vs nearest-even rounding of the exact value
    want = synth.bf16_bits(torch.from_numpy(ref).to(torch.bfloat16))
    diff = np.abs(yb_bits.astype(np.int32) - want.astype(np.int32))
    assert diff.max() <= 1, f"{what}: bf16 off by {diff.max()} ulp"
    assert (diff > 0).mean() < 1e-3


@pytest.mark.parametrize("m", [1, 8, 64])
def test_config2_all_sigma_stages(m):
    for stage in range(STAGES):
        sigma = q.aqn_sigma(stage, STAGES, SIGMA0, SIGMA1)
        out = _run(m, 3584, sigma, seed=1002, step=stage, layer=3, x_seed=50 + m)
        _check(*out, what=f"m={m} stage={stage}")


@pytest.mark.parametrize("m", [16, 256, 8192])
def test_config3_4_width_5120(m):
    out = _run(m, 5120, q.aqn_sigma(2, STAGES, SIGMA0, SIGMA1), seed=1003, step=2, layer=11, x_seed=60)
    _check(*out, what=f"m={m}")


@pytest.mark.parametrize("m,h", [(600, 8), (600, 1000), (517, 8192), (513, 8200), (600, 16384), (700, 37)])
def test_large_m_whole_rows(m, h):
    """Above 512 rows a workgroup takes whole rows (the vector-aligned widths
    here; 37 keeps the per-channel path): row groups with a ragged last one,
    the widest rows, and a width with pieces past the last full thread."""
    out = _run(m, h, 1e-2, seed=13, step=5, layer=2, x_seed=100 + h)
    _check(*out, what=f"m={m} h={h}")


@pytest.mark.parametrize("h", [1, 3, 37, 1000, 4095, 16384])
def test_ragged_widths(h):
    out = _run(3, h, 1e-2, seed=9, step=1, layer=0, x_seed=70 + h)
    _check(*out, what=f"h={h}")


def test_sigma_zero_and_strided_rows():
    out = _run(5, 512, 0.0, seed=1, step=0, layer=0, x_seed=80, ldx_pad=24)
    _check(*out, what="sigma=0")
    _, _, wn, _, _ = out
    w = synth.norm_weight_f32(512, seed=81).numpy()
    assert np.array_equal(wn, w)


def test_noise_depends_on_seed_step_layer_only():
    h = 2048
    base = _run(2, h, 1e-2, seed=5, step=3, layer=4, x_seed=90)[2]
    again = _run(7, h, 1e-2, seed=5, step=3, layer=4, x_seed=90)[2]
    assert np.array_equal(base, again)
    other = _run(2, h, 1e-2, seed=5, step=4, layer=4, x_seed=90)[2]
    assert not np.array_equal(base, other)


def test_bf16_output_only():
    m, h = 4, 3584
    x = synth.bf16_bits(synth.activation_bf16(m, h, seed=91))
    w = synth.norm_weight_f32(h, seed=92)
    yf, yb = q.aqn_rmsnorm(bits_to_gpu(x), w.to(dev()), EPS, 1e-3, 1, 2, 3, want_f32=False, want_bf16=True)
    torch.cuda.synchronize()
    assert yf is None
    ref, _ = oracle.aqn_rmsnorm(x, w.numpy(), EPS, float(np.float32(1e-3)), 1, 2, 3)
    want = synth.bf16_bits(torch.from_numpy(ref).to(torch.bfloat16))
    assert np.abs(gpu_bits(yb).astype(np.int32) - want.astype(np.int32)).max() <= 1
