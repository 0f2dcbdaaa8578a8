"""Pins of the oracle backward of the W4A16 + LoRA layer (dx, dA, dB).

Checked against: torch float64 autograd through the layer built on the
independent dequantization, and Euler's identity for maps that are linear in
one argument, which ties the backward to the (separately pinned) forward
oracle: <dx, x> = <dy, y>, and <dA, A> = <dB, B> = <dy, y - y_without_LoRA>.
"""
import numpy as np
import pytest
import torch

import oracle
from golden_tables import bf16_bits_to_f64, dequant_f64
from nvfp4_weight_only_quantize_amd import synth


def _case(m, n, k, r, seed):
    w = synth.weight_bf16(n, k, seed=seed, row_lognormal_sigma=0.5)
    packed, scales, s_t = oracle.nvfp4_quantize(synth.bf16_bits(w))
    x = synth.bf16_bits(synth.activation_bf16(m, k, seed=seed + 1, outlier_col_frac=0.01))
    dy = synth.bf16_bits(synth.activation_bf16(m, n, seed=seed + 2))
    a = b = None
    if r:
        a, b = synth.lora_bf16(n, k, r, seed=seed + 3)
        a, b = synth.bf16_bits(a), synth.bf16_bits(b)
    return dy, x, packed, scales, s_t, a, b


@pytest.mark.parametrize("shape", [(3, 40, 64, 8), (8, 96, 256, 16), (1, 16, 32, 4), (5, 48, 128, 0)])
def test_backward_matches_torch_autograd(shape):
    m, n, k, r = shape
    lam = 2.0
    dy, x, packed, scales, s_t, a, b = _case(m, n, k, r, seed=91 + k)
    dx, da, db = oracle.w4a16_lora_backward(dy, x, packed, scales, s_t, a, b, lam)
    xt = torch.from_numpy(bf16_bits_to_f64(x)).requires_grad_(True)
    wt = torch.from_numpy(dequant_f64(packed, scales, s_t))
    y = xt @ wt.T
    if r:
        at = torch.from_numpy(bf16_bits_to_f64(a)).requires_grad_(True)
        bt = torch.from_numpy(bf16_bits_to_f64(b)).requires_grad_(True)
        y = y + lam * ((xt @ at.T) @ bt.T)
    y.backward(torch.from_numpy(bf16_bits_to_f64(dy)))
    np.testing.assert_allclose(dx, xt.grad.numpy(), atol=1e-12 * np.abs(xt.grad.numpy()).max(), rtol=1e-10)
    if r:
        np.testing.assert_allclose(da, at.grad.numpy(), atol=1e-12 * np.abs(at.grad.numpy()).max(), rtol=1e-10)
        np.testing.assert_allclose(db, bt.grad.numpy(), atol=1e-12 * np.abs(bt.grad.numpy()).max(), rtol=1e-10)
    else:
        assert da is None and db is None


def test_backward_euler_identities_against_the_forward_oracle():
    m, n, k, r, lam = 4, 64, 256, 16, 1.5
    dy, x, packed, scales, s_t, a, b = _case(m, n, k, r, seed=101)
    dx, da, db = oracle.w4a16_lora_backward(dy, x, packed, scales, s_t, a, b, lam)
    y = oracle.w4a16_lora_gemm(x, packed, scales, s_t, a, b, lam)
    y0 = oracle.w4a16_lora_gemm(x, packed, scales, s_t)
    dyf = bf16_bits_to_f64(dy)
    inner = float((dyf * y).sum())
    lora = float((dyf * (y - y0)).sum())
    assert abs(float((dx * bf16_bits_to_f64(x)).sum()) - inner) <= 1e-9 * abs(inner)
    assert abs(float((da * bf16_bits_to_f64(a)).sum()) - lora) <= 1e-9 * abs(lora)
    assert abs(float((db * bf16_bits_to_f64(b)).sum()) - lora) <= 1e-9 * abs(lora)
