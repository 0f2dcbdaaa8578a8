"""Pins of the oracle AQN pieces: sigma schedule, Philox4x64-10 stream,
Gaussian noise and the noisy RMSNorm.

Checked against: the schedule's endpoints and constant ratio, numpy's
Philox (a library implementation of the same published generator), moment
and Kolmogorov-Smirnov tests of the Box-Muller output, torch's rms_norm at
sigma = 0, and the additive form of the noise.
"""
import math

import numpy as np
import pytest
import scipy.stats
import torch

import oracle
from nvfp4_weight_only_quantize_amd import synth


def test_sigma_schedule_endpoints_and_ratio():
    s0, s1, S = 1e-2, 5e-4, 10
    sig = [oracle.aqn_sigma(k, S, s0, s1) for k in range(S)]
    assert sig[0] == s0
    assert abs(sig[-1] - s1) <= 1e-15 * s1
    ratios = [sig[i + 1] / sig[i] for i in range(S - 1)]
    want = (s1 / s0) ** (1 / (S - 1))
    assert abs(want - 0.7168711641) < 1e-9
    for q in ratios:
        assert abs(q - want) <= 1e-13
    assert all(sig[i] > sig[i + 1] for i in range(S - 1))
    assert oracle.aqn_sigma(0, 1, s0, s1) == s0
    assert oracle.aqn_sigma(-3, S, s0, s1) == s0
    assert abs(oracle.aqn_sigma(99, S, s0, s1) - s1) <= 1e-15 * s1


def _numpy_philox_block(counter, key):
    """numpy increments the counter before each block, so start one below."""
    c = np.array(counter, dtype=np.uint64)
    prev = [(int(c[0]) - 1) & (2 ** 64 - 1), int(c[1]), int(c[2]), int(c[3])]
    if int(c[0]) == 0:  # borrow into the next words
        i = 1
        while True:
            prev[i] = (prev[i] - 1) & (2 ** 64 - 1)
            if prev[i] != 2 ** 64 - 1 or i == 3:
                break
            i += 1
    bg = np.random.Philox(counter=np.array(prev, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    return bg.random_raw(4)


@pytest.mark.parametrize("counter,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 0, 0, 0), (0, 0)),
    ((5, 7, 0, 0), (1234, 9)),
    ((0, 3, 0, 0), (2 ** 64 - 1, 2 ** 63)),
    ((2 ** 40 + 17, 2 ** 33, 5, 6), (0xDEADBEEF, 42)),
])
def test_philox_matches_numpy(counter, key):
    assert np.array_equal(oracle.philox4x64_10(counter, key), _numpy_philox_block(counter, key))


def test_noise_is_deterministic_and_gaussian():
    z = oracle.aqn_noise(seed=1002, step=3, layer=7, h=1 << 20)
    assert np.array_equal(z, oracle.aqn_noise(1002, 3, 7, 1 << 20))
    n = z.size
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1) < 5 * math.sqrt(2 / n)
    assert abs(scipy.stats.skew(z)) < 0.02
    assert abs(scipy.stats.kurtosis(z)) < 0.04
    assert scipy.stats.kstest(z, "norm").pvalue > 1e-3


def test_noise_streams_differ_across_step_layer_seed():
    h = 1 << 16
    base = oracle.aqn_noise(5, 0, 0, h)
    for other in (oracle.aqn_noise(5, 1, 0, h), oracle.aqn_noise(5, 0, 1, h), oracle.aqn_noise(6, 0, 0, h)):
        assert abs(np.corrcoef(base, other)[0, 1]) < 0.02
    # a prefix of a longer vector is the shorter vector (ragged H)
    assert np.array_equal(oracle.aqn_noise(5, 0, 0, 37), base[:37])


def _x(m, h, seed):
    return synth.bf16_bits(synth.activation_bf16(m, h, seed=seed, outlier_col_frac=0.005))


def test_sigma_zero_is_torch_rms_norm():
    m, h = 5, 3584
    x = _x(m, h, 1)
    w = synth.norm_weight_f32(h, seed=2).numpy()
    y, wn = oracle.aqn_rmsnorm(x, w, eps=1e-6, sigma=0.0, seed=1, step=0, layer=0)
    xd = synth.bits_to_bf16(x).to(torch.float64)
    ref = torch.nn.functional.rms_norm(xd, (h,), weight=torch.from_numpy(w.astype(np.float64)), eps=1e-6)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=0)
    assert np.array_equal(wn, w.astype(np.float64))


def test_noise_is_additive_on_the_norm_weight():
    m, h = 3, 1000
    x = _x(m, h, 3)
    w = synth.norm_weight_f32(h, seed=4).numpy()
    sigma = 1e-2
    y, wn = oracle.aqn_rmsnorm(x, w, 1e-6, sigma, seed=11, step=2, layer=5)
    z = oracle.aqn_noise(11, 2, 5, h)
    # (w + sigma z) - w cancels: allow one ulp of w
    np.testing.assert_allclose(wn - w.astype(np.float64), sigma * z, rtol=0, atol=4e-16)
    assert np.std(wn - w) == pytest.approx(sigma, rel=0.1)
    # and y is the plain RMSNorm of x with that weight
    np.testing.assert_allclose(y, oracle.rmsnorm(x, wn, 1e-6), rtol=1e-15)


def test_rmsnorm_rows_are_scale_invariant():
    m, h = 4, 512
    x = _x(m, h, 5)
    x2 = synth.bf16_bits(synth.bits_to_bf16(x).to(torch.float64).mul(8).to(torch.bfloat16))
    w = np.ones(h)
    y1 = oracle.rmsnorm(x, w, 1e-30)
    y2 = oracle.rmsnorm(x2, w, 1e-30)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)
    # rms of each output row is one when eps is negligible
    np.testing.assert_allclose(np.sqrt((y1 ** 2).mean(axis=1)), 1.0, rtol=1e-12)


def test_zero_row_gives_zero_output():
    x = np.zeros((2, 64), dtype=np.uint16)
    y, _ = oracle.aqn_rmsnorm(x, np.ones(64, dtype=np.float32), 1e-6, 1e-3, 0, 0, 0)
    assert np.all(y == 0)
