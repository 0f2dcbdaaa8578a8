"""Pins of the oracle quantizer variants: stochastic element rounding of
NVFP4 and the MXFP4 (OCP MX, block 32, E8M0 scale) format.

Stochastic rounding is checked against: numpy's Philox for the uniforms, an
exact-rational restatement of the rounding rule, its defining property (the
expected dequantized value is the input) over many seeds, neighbours-only
outputs, fixed grid values, and the unchanged block scales.  MXFP4 is checked
against an exact restatement of the OCP conversion (scale exponent from
frexp, nearest-even by brute force over the grid) and exact round trips.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from golden_tables import E2M1, E2M1_FRAC, E4M3, bf16_bits_to_f64, dequant_f64
from nvfp4_weight_only_quantize_amd import synth

GRID = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]


def _w(n, k, seed):
    return synth.bf16_bits(synth.weight_bf16(n, k, seed=seed, row_lognormal_sigma=0.5))


def _numpy_uniform(seed, e):
    # counter (e/4, 0, 1, 0), key (seed, 0); numpy increments before each block
    ctr = [e // 4, 0, 1, 0]
    prev = list(ctr)
    prev[0] = (prev[0] - 1) % 2 ** 64
    if ctr[0] == 0:
        prev[1] = (prev[1] - 1) % 2 ** 64
        if ctr[1] == 0:
            prev[2] = (prev[2] - 1) % 2 ** 64
    bg = np.random.Philox(counter=np.array(prev, dtype=np.uint64), key=np.array([seed, 0], dtype=np.uint64))
    r = bg.random_raw(4)
    return float(int(r[e % 4]) >> 40) * 2.0 ** -24


@pytest.mark.parametrize("seed,e", [(0, 0), (0, 3), (7, 4), (2 ** 64 - 1, 1234567), (99, 2 ** 33 + 2)])
def test_sr_uniform_matches_numpy_philox(seed, e):
    assert oracle.sr_uniform(seed, e) == _numpy_uniform(seed, e)


def _sr_codes(w_bits, seed, flags=0):
    packed, scales, s_t = oracle.nvfp4_quantize(w_bits, flags=flags, stochastic_seed=seed)
    n, k = w_bits.shape
    codes = np.empty((n, k), dtype=np.int64)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    return codes, scales, s_t


@pytest.mark.parametrize("flags", [0, 1])
def test_sr_rule_exact_rationals(flags):
    n, k, seed = 6, 64, 321
    w = _w(n, k, seed=11)
    codes, scales, s_t = _sr_codes(w, seed, flags)
    _, det_scales, det_st = oracle.nvfp4_quantize(w, flags=flags)
    assert np.array_equal(scales, det_scales) and s_t == det_st
    wf = bf16_bits_to_f64(w)
    st = Fraction(float(s_t))
    for r in range(n):
        for c in range(k):
            S = Fraction(E4M3[scales[r, c // 16]]) * st
            a = Fraction(abs(float(wf[r, c])))
            u = Fraction(oracle.sr_uniform(seed, r * k + c))
            if S == 0:
                mag = 0
            else:
                v = a / S
                lo = max(i for i in range(8) if GRID[i] <= v)
                mag = lo if lo == 7 else (lo + 1 if u < (v - GRID[lo]) / (GRID[lo + 1] - GRID[lo]) else lo)
            sign = int(np.signbit(wf[r, c]))
            assert codes[r, c] == (sign << 3) | mag, (r, c)


def test_sr_is_unbiased_and_picks_neighbours():
    n, k = 2, 32
    w = _w(n, k, seed=12)
    wf = bf16_bits_to_f64(w)
    seeds = 400
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    total = np.zeros((n, k))
    _, scales0, s_t = _sr_codes(w, 0)
    S = np.array([[E4M3[scales0[r, c // 16]] * float(s_t) for c in range(k)] for r in range(n)])
    v = np.abs(wf) / S
    idx = np.searchsorted(grid, v, side="right") - 1
    lo, hi = grid[idx], grid[np.minimum(idx + 1, 7)]
    for sd in range(seeds):
        codes, scales, _ = _sr_codes(w, 1000 + sd)
        assert np.array_equal(scales, scales0)
        deq = np.array([[E2M1[codes[r, c]] for c in range(k)] for r in range(n)]) * S
        # each output is one of the two grid neighbours of |w| / S
        got = np.abs(deq) / S
        assert np.all((got == lo) | (got == hi))
        total += deq
    # one draw has standard deviation at most (hi - lo) S / 2, so the mean of
    # the draws lies within 5 of those over sqrt(draws) of w (nearest-even
    # rounding would miss by up to half a gap)
    mean = total / seeds
    assert np.all(np.abs(mean - wf) <= 5 * (hi - lo) * S / 2 / math.sqrt(seeds) + 1e-30)


def test_sr_keeps_grid_values_and_differs_across_seeds():
    # a block whose values lie on the grid of its own scale stays exact
    k = 16
    vals = np.array([0, .5, -1, 1.5, 2, -3, 4, 6, 6, -6, 0.5, 1, -2, 3, 4, 1.5]) * 2.0 ** -3
    bits = synth.bf16_bits(__import__("torch").tensor(vals, dtype=__import__("torch").float32).to(
        __import__("torch").bfloat16)).reshape(1, k)
    for sd in (1, 2, 3):
        assert np.array_equal(_sr_codes(bits, sd)[0], _sr_codes(bits, 1)[0])
    w = _w(8, 256, seed=13)
    assert not np.array_equal(_sr_codes(w, 1)[0], _sr_codes(w, 2)[0])


# ----------------------------------------------------------------- MXFP4 --
def _mx_ref(w_bits):
    wf = bf16_bits_to_f64(w_bits)
    n, k = wf.shape
    codes = np.zeros((n, k), dtype=np.int64)
    scales = np.zeros((n, k // 32), dtype=np.int64)
    for r in range(n):
        for b in range(k // 32):
            blk = wf[r, 32 * b:32 * b + 32]
            amax = float(np.abs(blk).max())
            if amax == 0:
                sc = 0
            else:
                _, ex = math.frexp(amax)
                sc = min(max(ex - 1 - 2 + 127, 0), 254)
            scales[r, b] = sc
            X = Fraction(2) ** (sc - 127)
            for i, v in enumerate(blk):
                a = Fraction(abs(float(v))) / X
                # nearest grid value, ties to the even code, above 6 -> 6
                best = min(range(8), key=lambda j: (abs(GRID[j] - a), j & 1))
                codes[r, 32 * b + i] = (int(np.signbit(v)) << 3) | best
    return codes, scales


@pytest.mark.parametrize("shape,seed", [((4, 64), 21), ((3, 128), 22), ((1, 32), 23)])
def test_mxfp4_matches_the_ocp_definition(shape, seed):
    w = _w(*shape, seed=seed)
    packed, scales = oracle.mxfp4_quantize(w)
    codes = np.empty(shape, dtype=np.int64)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    ref_codes, ref_scales = _mx_ref(w)
    assert np.array_equal(scales, ref_scales)
    assert np.array_equal(codes, ref_codes)


def test_mxfp4_round_trip_and_zero_block():
    import torch
    rng = np.random.default_rng(5)
    k = 64
    # block 0: grid values times 2^-5 (amax 6 * 2^-5 -> scale 2^(2-5-2) ... exact); block 1: zeros
    g = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    vals = np.concatenate([g[rng.integers(0, 8, 32)] * rng.choice([-1, 1], 32) * 2.0 ** -5, np.zeros(32)])
    vals[0] = 6 * 2.0 ** -5  # the block amax sits on the grid top
    bits = synth.bf16_bits(torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)).reshape(1, k)
    packed, scales = oracle.mxfp4_quantize(bits)
    codes = np.empty(k, dtype=np.int64)
    codes[0::2] = packed[0] & 15
    codes[1::2] = packed[0] >> 4
    X = [2.0 ** (int(s) - 127) for s in scales[0]]
    deq = np.array([E2M1[c] * X[i // 32] for i, c in enumerate(codes)])
    assert np.array_equal(deq, vals)
    assert scales[0, 1] == 0
