"""Independent decoding tables used by the oracle pins.

E2M1 values come from the cited golden fixture; E4M3 values come from
PyTorch's float8_e4m3fn dtype (a library routine), not from the oracle.
"""
import os
from fractions import Fraction

import numpy as np
import torch

_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e2m1_table():
    vals = {}
    with open(os.path.join(_GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    assert sorted(vals) == list(range(16))
    return [vals[c] for c in range(16)]


def e4m3_table():
    """float value of every E4M3 byte, via torch's float8_e4m3fn."""
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return b.view(torch.float8_e4m3fn).to(torch.float64).numpy()


E2M1 = e2m1_table()
E4M3 = e4m3_table()
E2M1_FRAC = [Fraction(v) for v in E2M1]


def bf16_bits_to_f64(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits_exact(v):
    """float64 values that are exactly representable in BF16 -> bit patterns."""
    v = np.asarray(v, dtype=np.float64)
    f = v.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v, equal_nan=True) or np.all(np.isnan(v) == np.isnan(f))
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def dequant_f64(packed, scales, s_t):
    """what[n, k] = e2m1 * e4m3 * s_t from the independent tables."""
    packed = np.asarray(packed, dtype=np.uint8)
    n, kh = packed.shape
    codes = np.empty((n, kh * 2), dtype=np.int64)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    e2 = np.array(E2M1)[codes]
    sc = E4M3[np.asarray(scales, dtype=np.int64)]
    return e2 * np.repeat(sc, 16, axis=1) * float(s_t)
