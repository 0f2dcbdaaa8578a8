"""Pins of the oracle W4A16 + LoRA layer (fp64).

Checked against: exact-rational brute force on tiny shapes, torch float64
matmul on a dequantization built from independent tables, one-hot inputs,
the B = 0 / r = 0 / W = 0 reductions, exact scaling by two, row sampling,
and the block-diagonal (fused gate/up) LoRA identity.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from golden_tables import E2M1_FRAC, E4M3, bf16_bits_to_f64, dequant_f64
from nvfp4_weight_only_quantize_amd import synth


def _layer(m, n, k, r, seed, x_outliers=0.0):
    w = synth.weight_bf16(n, k, seed=seed, row_lognormal_sigma=0.5)
    packed, scales, s_t = oracle.nvfp4_quantize(synth.bf16_bits(w))
    x = synth.bf16_bits(synth.activation_bf16(m, k, seed=seed + 1, outlier_col_frac=x_outliers))
    if r:
        a, b = synth.lora_bf16(n, k, r, seed=seed + 2)
        a, b = synth.bf16_bits(a), synth.bf16_bits(b)
    else:
        a = b = None
    return x, packed, scales, s_t, a, b


def _torch_ref(x, packed, scales, s_t, a, b, lam):
    xd = torch.from_numpy(bf16_bits_to_f64(x))
    wd = torch.from_numpy(dequant_f64(packed, scales, s_t))
    y = xd @ wd.T
    if a is not None:
        ad = torch.from_numpy(bf16_bits_to_f64(a))
        bd = torch.from_numpy(bf16_bits_to_f64(b))
        y = y + lam * ((xd @ ad.T) @ bd.T)
    return y.numpy()


@pytest.mark.parametrize("shape", [(1, 16, 32, 4), (3, 24, 32, 2), (2, 8, 16, 1), (4, 32, 32, 0)])
def test_rational_brute_force(shape):
    m, n, k, r = shape
    x, packed, scales, s_t, a, b = _layer(m, n, k, r, seed=31 + m + n)
    lam = 2.0
    y = oracle.w4a16_lora_gemm(x, packed, scales, s_t, a, b, lam)
    xf = [[Fraction(float(v)) for v in row] for row in bf16_bits_to_f64(x)]
    codes = np.empty((n, k), dtype=np.int64)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    st = Fraction(float(s_t))
    wf = [[E2M1_FRAC[codes[i, j]] * Fraction(E4M3[scales[i, j // 16]]) * st for j in range(k)]
          for i in range(n)]
    if r:
        af = [[Fraction(float(v)) for v in row] for row in bf16_bits_to_f64(a)]
        bf = [[Fraction(float(v)) for v in row] for row in bf16_bits_to_f64(b)]
    for i in range(m):
        t = [sum(xf[i][j] * af[q][j] for j in range(k)) for q in range(r)] if r else []
        for o in range(n):
            exact = sum(xf[i][j] * wf[o][j] for j in range(k))
            if r:
                exact += Fraction(lam) * sum(t[q] * bf[o][q] for q in range(r))
            got = Fraction(float(y[i, o]))
            tol = Fraction(1, 10 ** 12) * max(abs(exact), Fraction(1, 10 ** 30))
            assert abs(got - exact) <= tol, (i, o, float(got), float(exact))


@pytest.mark.parametrize("shape", [(5, 96, 256, 16), (64, 40, 512, 32), (1, 512, 2048, 8)])
def test_matches_torch_float64(shape):
    m, n, k, r = shape
    x, packed, scales, s_t, a, b = _layer(m, n, k, r, seed=41 + k, x_outliers=0.005)
    y = oracle.w4a16_lora_gemm(x, packed, scales, s_t, a, b, 2.0, threads=3)
    ref = _torch_ref(x, packed, scales, s_t, a, b, 2.0)
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_one_hot_rows_pick_weight_columns():
    m, n, k, r = 4, 48, 64, 4
    _, packed, scales, s_t, a, b = _layer(1, n, k, r, seed=51)
    cols = [0, 17, 33, 63]
    x = np.zeros((m, k), dtype=np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = 0x3F80  # 1.0
    lam = 0.5
    y = oracle.w4a16_lora_gemm(x, packed, scales, s_t, a, b, lam)
    wd = dequant_f64(packed, scales, s_t)
    ad, bd = bf16_bits_to_f64(a), bf16_bits_to_f64(b)
    for i, c in enumerate(cols):
        want = wd[:, c] + lam * (bd @ ad[:, c])
        np.testing.assert_allclose(y[i], want, rtol=1e-14, atol=1e-300)


def test_zero_lora_and_zero_weight_reductions():
    m, n, k, r = 3, 40, 128, 8
    x, packed, scales, s_t, a, b = _layer(m, n, k, r, seed=61)
    base = oracle.w4a16_lora_gemm(x, packed, scales, s_t)
    zb = np.zeros_like(b)
    assert np.array_equal(oracle.w4a16_lora_gemm(x, packed, scales, s_t, a, zb, 2.0), base)
    # W = 0: codes and scales zero -> LoRA term only
    zp, zs = np.zeros_like(packed), np.zeros_like(scales)
    lora_only = oracle.w4a16_lora_gemm(x, zp, zs, s_t, a, b, 2.0)
    full = oracle.w4a16_lora_gemm(x, packed, scales, s_t, a, b, 2.0)
    np.testing.assert_allclose(full, base + lora_only, rtol=1e-12, atol=1e-14)


def test_doubling_x_doubles_y_exactly():
    m, n, k, r = 2, 32, 256, 4
    x, packed, scales, s_t, a, b = _layer(m, n, k, r, seed=71)
    x2 = synth.bf16_bits(synth.bits_to_bf16(x).to(torch.float64).mul(2).to(torch.bfloat16))
    y1 = oracle.w4a16_lora_gemm(x, packed, scales, s_t, a, b, 2.0)
    y2 = oracle.w4a16_lora_gemm(x2, packed, scales, s_t, a, b, 2.0)
    assert np.array_equal(2 * y1, y2)


def test_row_sampling_equals_full_rows():
    m, n, k, r = 9, 24, 128, 4
    x, packed, scales, s_t, a, b = _layer(m, n, k, r, seed=81)
    full = oracle.w4a16_lora_gemm(x, packed, scales, s_t, a, b, 2.0)
    rows = [8, 0, 5]
    part = oracle.w4a16_lora_gemm(x, packed, scales, s_t, a, b, 2.0, rows=rows)
    assert np.array_equal(part, full[rows])


def test_block_diagonal_lora_equals_two_separate_loras():
    # fused gate/up: one NVFP4 tensor [2N, K], A = [A_g; A_u], B block-diagonal
    m, n, k, r = 3, 32, 256, 4
    x, packed, scales, s_t, _, _ = _layer(m, 2 * n, k, 0, seed=91)
    ag, bg = (synth.bf16_bits(t) for t in synth.lora_bf16(n, k, r, seed=92))
    au, bu = (synth.bf16_bits(t) for t in synth.lora_bf16(n, k, r, seed=93))
    a = np.concatenate([ag, au], axis=0)
    b = np.zeros((2 * n, 2 * r), dtype=np.uint16)
    b[:n, :r] = bg
    b[n:, r:] = bu
    lam = 2.0
    fused = oracle.w4a16_lora_gemm(x, packed, scales, s_t, a, b, lam)
    base = oracle.w4a16_lora_gemm(x, packed, scales, s_t)
    g = oracle.w4a16_lora_gemm(x, packed[:n], scales[:n], s_t, ag, bg, lam)
    u = oracle.w4a16_lora_gemm(x, packed[n:], scales[n:], s_t, au, bu, lam)
    sep = np.concatenate([g, u], axis=1)
    np.testing.assert_allclose(fused, sep, rtol=1e-12, atol=1e-14 * np.abs(base).max())


# ---- fp64 activations and the RMSNorm + layer composite ----
@pytest.mark.parametrize("shape", [(3, 40, 256, 8), (16, 64, 512, 0)])
def test_fp64_activations_match_torch_float64(shape):
    # activations that are not BF16 values (a norm's output before rounding)
    m, n, k, r = shape
    _, packed, scales, s_t, a, b = _layer(1, n, k, r, seed=61 + k)
    x = np.random.default_rng(62).standard_normal((m, k)) * np.exp(np.random.default_rng(63).standard_normal(k))
    y = oracle.w4a16_lora_gemm(None, packed, scales, s_t, a, b, 1.5, threads=2, x_f64=x)
    xd = torch.from_numpy(x)
    ref = xd @ torch.from_numpy(dequant_f64(packed, scales, s_t)).T
    if r:
        ref = ref + 1.5 * ((xd @ torch.from_numpy(bf16_bits_to_f64(a)).T) @ torch.from_numpy(bf16_bits_to_f64(b)).T)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-10, atol=1e-12 * np.abs(ref.numpy()).max())


def test_rmsnorm_layer_composite_matches_torch():
    # RMSNorm (torch's rms_norm in fp64, scale vector w) followed by the layer
    # (torch fp64 matmul on the independent dequantization)
    m, n, k, r = 5, 48, 256, 16
    x, packed, scales, s_t, a, b = _layer(m, n, k, r, seed=71, x_outliers=0.01)
    w = (1.0 + 0.1 * np.random.default_rng(72).standard_normal(k)).astype(np.float32)
    y = oracle.rmsnorm_w4a16_lora_gemm(x, w, 1e-6, packed, scales, s_t, a, b, 2.0)
    xn = torch.nn.functional.rms_norm(torch.from_numpy(bf16_bits_to_f64(x)), (k,),
                                      weight=torch.from_numpy(w.astype(np.float64)), eps=1e-6)
    ref = xn @ torch.from_numpy(dequant_f64(packed, scales, s_t)).T
    ref = ref + 2.0 * ((xn @ torch.from_numpy(bf16_bits_to_f64(a)).T) @ torch.from_numpy(bf16_bits_to_f64(b)).T)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-9, atol=1e-12 * np.abs(ref.numpy()).max())


def test_rmsnorm_layer_composite_row_scale_invariance():
    # RMSNorm makes each output row invariant under scaling its input row by 2^j
    m, n, k, r = 3, 32, 128, 4
    x, packed, scales, s_t, a, b = _layer(m, n, k, r, seed=81)
    w = np.linspace(0.5, 1.5, k).astype(np.float32)
    y = oracle.rmsnorm_w4a16_lora_gemm(x, w, 1e-30, packed, scales, s_t, a, b, 2.0)
    xs = bf16_bits_to_f64(x) * np.array([[4.0], [0.25], [1.0]])
    xs_bits = synth.bf16_bits(torch.from_numpy(xs).to(torch.bfloat16))
    y2 = oracle.rmsnorm_w4a16_lora_gemm(xs_bits, w, 1e-30, packed, scales, s_t, a, b, 2.0)
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-14 * np.abs(y).max())
