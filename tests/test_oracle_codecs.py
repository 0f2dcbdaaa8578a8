"""Pins of the oracle's element codecs and rounding helpers.

Each check compares the oracle with something other than itself: the cited
E2M1 table, PyTorch's float8_e4m3fn decode and float32->e4m3fn cast (library
routines), or brute force with exact rationals.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from golden_tables import E2M1, E2M1_FRAC, E4M3


def test_e2m1_all_codes_match_golden_table():
    for c in range(16):
        got = oracle.e2m1_decode(c)
        assert got == E2M1[c], c
        assert math.copysign(1.0, got) == math.copysign(1.0, E2M1[c]), c
    assert max(abs(v) for v in E2M1) == 6.0


def test_e4m3_all_bytes_match_torch():
    for b in range(256):
        got = oracle.e4m3_decode(b)
        want = E4M3[b]
        if math.isnan(want):
            assert math.isnan(got), b
        else:
            assert got == want, (b, got, want)
            assert math.copysign(1.0, got) == math.copysign(1.0, want), b
    assert np.nanmax(E4M3) == 448.0
    assert [b for b in range(256) if math.isnan(E4M3[b])] == [0x7F, 0xFF]


def _roundup_brute(amax_b: Fraction, s_t: Fraction) -> int:
    for code in range(0x7F):  # 0x00..0x7E, increasing values
        if Fraction(E4M3[code]) * 6 * s_t >= amax_b:
            return code
    return 0x7E


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_e4m3_round_up_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    for _ in range(400):
        s_t = np.float32(2.0 ** rng.uniform(-30, 10) * rng.uniform(1, 2))
        # amax spanning below, inside and above the E4M3 range relative to 6 s_t
        t = 2.0 ** rng.uniform(-14, 10)
        amax = float(torch.tensor(t * 6.0 * float(s_t), dtype=torch.float64).to(torch.bfloat16))
        want = _roundup_brute(Fraction(amax), Fraction(float(s_t)))
        assert oracle.e4m3_block_scale_code(amax, float(s_t), oracle.SCALE_ROUND_UP) == want


def test_e4m3_round_up_exact_hits_and_neighbours():
    s_t = 2.0 ** -7
    for code in range(1, 0x7F):
        v = E4M3[code]
        amax = v * 6 * s_t  # exact: block amax lands on an E4M3 value
        assert oracle.e4m3_block_scale_code(amax, s_t, oracle.SCALE_ROUND_UP) == code
        # a hair above goes to the next code (saturating at 448)
        above = np.nextafter(amax, np.inf)
        assert oracle.e4m3_block_scale_code(above, s_t, oracle.SCALE_ROUND_UP) == min(code + 1, 0x7E)
    assert oracle.e4m3_block_scale_code(0.0, s_t, oracle.SCALE_ROUND_UP) == 0


def _torch_e4m3_rne(t: np.ndarray) -> np.ndarray:
    return torch.from_numpy(t.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_rne_matches_torch_cast():
    # with s_t a power of two and amax = 6 t s_t, the exact quotient t* = t is a
    # float32, so the nearest-even scale must equal torch's float32->e4m3fn cast
    rng = np.random.default_rng(7)
    ts = [np.float32(E4M3[c]) for c in range(0x7F)]
    # every midpoint between neighbours (ties) and a float32 ulp either side
    mids = [np.float32((E4M3[c] + E4M3[c + 1]) / 2) for c in range(0x7E)]
    ts += mids + [np.nextafter(m, np.float32(0)) for m in mids] + [np.nextafter(m, np.float32(1e9)) for m in mids]
    ts += list(np.float32(2.0 ** rng.uniform(-12, np.log2(448), size=4000)))
    ts += [np.float32(2.0 ** -10), np.float32(2.0 ** -10 * 1.0000001), np.float32(1e-6), np.float32(0.0)]
    ts = np.array([t for t in ts if t <= 448.0], dtype=np.float32)
    want = _torch_e4m3_rne(ts)
    for s_exp in (-8, 0, 5):
        s_t = 2.0 ** s_exp
        for t, w in zip(ts, want):
            amax = 6.0 * float(t) * s_t  # exact in float64
            got = oracle.e4m3_block_scale_code(amax, s_t, oracle.SCALE_RNE)
            assert got == int(w), (float(t), s_t, got, int(w))


def test_e4m3_rne_saturates():
    s_t = 1.0
    assert oracle.e4m3_block_scale_code(6 * 460.0, s_t, oracle.SCALE_RNE) == 0x7E
    assert oracle.e4m3_block_scale_code(6 * 1e6, s_t, oracle.SCALE_RNE) == 0x7E
    assert oracle.e4m3_block_scale_code(6 * 1e6, s_t, oracle.SCALE_ROUND_UP) == 0x7E


def _e2m1_brute(w: float, S: Fraction) -> int:
    sign = 1 if math.copysign(1.0, w) < 0 else 0
    if S == 0:
        return sign << 3
    v = abs(Fraction(w)) / S
    best = None
    for code in range(8):
        d = abs(v - E2M1_FRAC[code])
        key = (d, code & 1)  # nearest; on a tie the even code
        if best is None or key < best[0]:
            best = (key, code)
    return (sign << 3) | best[1]


def test_e2m1_code_at_every_midpoint_and_neighbour():
    for S in (Fraction(1), Fraction(3, 64), Fraction(448) * Fraction(1, 2 ** 20),
              Fraction(E4M3[9]) * Fraction(float(np.float32(0.0123456))) ):
        Sf = float(S)
        assert Fraction(Sf) == S
        for mid in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
            exact = float(Fraction(mid) * S)
            assert Fraction(exact) == Fraction(mid) * S
            for w in (exact, np.nextafter(exact, 0.0), np.nextafter(exact, np.inf)):
                for sgn in (1.0, -1.0):
                    ww = sgn * float(w)
                    assert oracle.e2m1_code(ww, Sf) == _e2m1_brute(ww, S), (ww, Sf)
        for w in (0.0, -0.0, 6.0 * Sf, 7.0 * Sf, 1e30, -1e30):
            assert oracle.e2m1_code(w, Sf) == _e2m1_brute(w, S)


def test_e2m1_code_random_against_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(3000):
        S = Fraction(E4M3[int(rng.integers(1, 0x7F))]) * Fraction(float(np.float32(rng.uniform(1e-3, 1))))
        w = float(rng.normal() * float(S) * 3)
        assert oracle.e2m1_code(w, float(S)) == _e2m1_brute(w, S)


def test_zero_scale_gives_signed_zero_codes():
    assert oracle.e2m1_code(1.0, 0.0) == 0
    assert oracle.e2m1_code(-1.0, 0.0) == 8
    assert oracle.e2m1_code(-0.0, 1.0) == 8


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 1 << 16, 37, dtype=np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_decode(int(b)) for b in bits])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
