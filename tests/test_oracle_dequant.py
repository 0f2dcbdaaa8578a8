"""Oracle NVFP4 -> BF16 dequantization and its BF16 rounding, pinned without
the oracle's own arithmetic.

- The exact values equal e2m1 x e4m3 x s_t from the independent tables
  (golden E2M1 fixture, torch's float8_e4m3fn), and the nibble order (even
  element in the low nibble) is checked one code at a time.
- The rounding is checked against brute force over the whole table of finite
  BF16 values (nearest magnitude, ties to the even code, IEEE overflow to
  infinity from half a step past the largest value), and on hand-worked ties.
"""
import numpy as np
import pytest

import oracle
from golden_tables import dequant_f64

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _bf16_values():
    """float64 value of every non-negative finite BF16 code 0 .. 0x7F7F."""
    codes = np.arange(0x7F80, dtype=np.uint32)
    return (codes << 16).view(np.float32).astype(np.float64)


def _brute_nearest_even(v):
    tab = _bf16_values()
    ext = np.append(tab, 2.0 ** 128)  # one step past the largest finite value
    out = np.empty(len(v), dtype=np.uint16)
    for i, x in enumerate(v):
        a = abs(x)
        hi = int(np.searchsorted(ext, a, side="left"))  # first code with value >= a
        if hi == len(ext) or ext[hi] == a:  # at or past 2^128: infinity; else exact
            c = min(hi, len(ext) - 1)
        else:
            lo = hi - 1
            da, db = a - ext[lo], ext[hi] - a
            c = lo if da < db else hi if db < da else (lo if lo % 2 == 0 else hi)
        out[i] = c | (0x8000 if np.signbit(x) else 0)
    return out


def test_rounding_hand_ties_and_ends():
    cases = [
        (1.0, 0x3F80), (1 + 2 ** -8, 0x3F80), (1 + 3 * 2 ** -8, 0x3F82), (1 + 2 ** -8 + 2 ** -30, 0x3F81),
        (-(1 + 2 ** -8), 0xBF80), (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000), (3 * 2.0 ** -134, 0x0002),
        (-(2.0 ** -134) * 1.0000001, 0x8001), (0.0, 0x0000), (-0.0, 0x8000),
        (float.fromhex("0x1.feffffffffp127"), 0x7F7F), (float.fromhex("0x1.ff0p127"), 0x7F80), (1e300, 0x7F80),
    ]
    for v, want in cases:
        assert oracle.bf16_nearest_even(v) == want, (v, hex(oracle.bf16_nearest_even(v)), hex(want))
    assert oracle.bf16_nearest_even(float("nan")) & 0x7FFF > 0x7F80


def test_rounding_against_brute_force():
    rng = np.random.default_rng(41)
    v = np.concatenate([
        rng.standard_normal(3000) * np.exp2(rng.integers(-140, 128, 3000)),
        # exact midpoints between neighbouring BF16 values, and a hair either side
        (lambda t: np.concatenate([t, np.nextafter(t, 0), np.nextafter(t, np.inf)]))(
            (lambda tab, i: (tab[i] + tab[i + 1]) / 2)(_bf16_values(), rng.integers(0, 0x7F7E, 800))),
    ])
    v = v * np.where(rng.random(len(v)) < 0.5, -1.0, 1.0)
    got = np.array([oracle.bf16_nearest_even(float(x)) for x in v], dtype=np.uint16)
    np.testing.assert_array_equal(got, _brute_nearest_even(v))


@pytest.mark.parametrize("s_t", [1.0, 0.0123, 3.0e-41, 2.5e36])
def test_dequantize_values_match_independent_tables(s_t):
    rng = np.random.default_rng(7)
    n, k = 9, 96
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (n, k // 16), dtype=np.uint8)
    f64, bits = oracle.nvfp4_dequantize(packed, scales, np.float32(s_t))
    ref = dequant_f64(packed, scales, np.float32(s_t))
    np.testing.assert_array_equal(f64, ref)
    np.testing.assert_array_equal(bits, _brute_nearest_even(ref.ravel()).reshape(n, k))


def test_nibble_order_and_scale_index():
    # one non-zero code at a time: element j of row 1 lands at column j
    n, k = 2, 32
    for j in (0, 1, 15, 16, 31):
        packed = np.zeros((n, k // 2), dtype=np.uint8)
        packed[1, j // 2] = 0x2 << (4 * (j % 2))  # code 2 = 1.0
        scales = np.full((n, k // 16), 0x38, dtype=np.uint8)  # E4M3 1.0
        scales[1, 1] = 0x40  # 2.0 for the second block of row 1
        f64, bits = oracle.nvfp4_dequantize(packed, scales, np.float32(0.5))
        want = np.zeros((n, k))
        want[1, j] = 0.5 * (2.0 if j >= 16 else 1.0)
        np.testing.assert_array_equal(f64, want)
        assert bits[1, j] == (0x3F80 if j >= 16 else 0x3F00)


def test_exact_when_representable():
    # s_t a power of two: every value is exact in BF16, so the bits decode to it
    rng = np.random.default_rng(8)
    packed = rng.integers(0, 256, (4, 64), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (4, 8), dtype=np.uint8)
    f64, bits = oracle.nvfp4_dequantize(packed, scales, np.float32(2.0 ** -20))
    dec = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(dec, f64)
