"""CPU oracle for the NVFP4 W4A16 + LoRA layer and the AQN RMSNorm.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package; the product path
(the HIP library and its binding) never does, and shares no code with it.

The arithmetic lives in ``qerl_oracle.c`` (plain C, fp64, exact where the
definition is exact).  This module only builds/loads that library and
marshals numpy arrays.  Sources are cited in the C file; in short:

* quantizer -- block scaling of the cuDNN formula quoted on the page "QeRL:
  NVFP4-Quantized Reinforcement Learning -- Redefining Efficiency in AI
  Training and Inference", section "NVFP4: NVIDIA's FP4 Format";
* W4A16 + LoRA layer -- same page, sections "LoRA (Low-Rank Adaptation)" and
  "Implementation and Practical Details"; the "NVlabs/QeRL" README,
  "Acknowledgement" (NVFP4 x BF16 rollout kernel);
* AQN RMSNorm -- "Paper 2510.11696 -- QeRL: Beyond Efficiency", "Summary";
  README "Hints for QeRL training" item 3 (sigma_start, sigma_end,
  num_stages).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qerl_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libqerl_oracle.so")
# a separately built copy of the same source (the sanitizer run of the tests)
_LIB_OVERRIDE = os.environ.get("QERL_ORACLE_LIB")

SCALE_ROUND_UP = 0
SCALE_RNE = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=gnu11",
               "-Wall", "-shared", "-fPIC", "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64, i32, u32, u64, dbl, flt = (ctypes.c_int64, ctypes.c_int, ctypes.c_uint,
                                    ctypes.c_uint64, ctypes.c_double, ctypes.c_float)
    lib.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_decode.restype = dbl
    lib.oracle_e2m1_decode.argtypes = [i32]
    lib.oracle_e2m1_decode.restype = dbl
    lib.oracle_e4m3_decode.argtypes = [i32]
    lib.oracle_e4m3_decode.restype = dbl
    lib.oracle_e4m3_block_scale_code.argtypes = [dbl, flt, u32]
    lib.oracle_e4m3_block_scale_code.restype = i32
    lib.oracle_e2m1_code.argtypes = [dbl, dbl]
    lib.oracle_e2m1_code.restype = i32
    lib.oracle_nvfp4_quantize.argtypes = [P, i64, i64, i64, P, u32, P, P, P, i32]
    lib.oracle_nvfp4_quantize.restype = i32
    lib.oracle_w4a16_lora_gemm.argtypes = [P, i64, i64, i64, P, P, flt, i64, P, P, i32, flt,
                                           P, i64, P, i32]
    lib.oracle_w4a16_lora_gemm.restype = i32
    lib.oracle_nvfp4_quantize_sr.argtypes = [P, i64, i64, i64, P, u32, u64, P, P, P, i32]
    lib.oracle_nvfp4_quantize_sr.restype = i32
    lib.oracle_sr_uniform.argtypes = [u64, i64]
    lib.oracle_sr_uniform.restype = dbl
    lib.oracle_e2m1_sr_mag.argtypes = [dbl, dbl, dbl]
    lib.oracle_e2m1_sr_mag.restype = i32
    lib.oracle_mxfp4_quantize.argtypes = [P, i64, i64, i64, P, P]
    lib.oracle_mxfp4_quantize.restype = i32
    lib.oracle_bf16_nearest_even.argtypes = [dbl]
    lib.oracle_bf16_nearest_even.restype = ctypes.c_uint16
    lib.oracle_nvfp4_dequantize.argtypes = [P, P, flt, i64, i64, P, P]
    lib.oracle_nvfp4_dequantize.restype = i32
    lib.oracle_w4a16_lora_backward.argtypes = [P, P, i64, i64, i64, P, P, flt, P, P, i32, flt, P, P, P, i32]
    lib.oracle_w4a16_lora_backward.restype = i32
    lib.oracle_w4a16_lora_gemm_f64.argtypes = lib.oracle_w4a16_lora_gemm.argtypes
    lib.oracle_w4a16_lora_gemm_f64.restype = i32
    lib.oracle_aqn_sigma.argtypes = [i32, i32, dbl, dbl]
    lib.oracle_aqn_sigma.restype = dbl
    lib.oracle_philox4x64_10.argtypes = [P, P, P]
    lib.oracle_philox4x64_10.restype = None
    lib.oracle_aqn_noise.argtypes = [u64, u64, u32, i64, P]
    lib.oracle_aqn_noise.restype = None
    lib.oracle_rmsnorm.argtypes = [P, i64, i64, i64, P, dbl, P]
    lib.oracle_rmsnorm.restype = i32
    lib.oracle_aqn_rmsnorm.argtypes = [P, i64, i64, i64, P, dbl, dbl, u64, u64, u32, P, P]
    lib.oracle_aqn_rmsnorm.restype = i32
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _bits16(a) -> np.ndarray:
    """Accept a uint16 array of BF16 bit patterns (or int16) and return uint16 C-order."""
    a = np.asarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected BF16 bit patterns as uint16")
    return a


# ----------------------------------------------------------------- codecs --
def bf16_decode(bits: int) -> float:
    return _load().oracle_bf16_decode(int(bits) & 0xFFFF)


def e2m1_decode(code: int) -> float:
    return _load().oracle_e2m1_decode(int(code))


def e4m3_decode(byte: int) -> float:
    return _load().oracle_e4m3_decode(int(byte))


def e4m3_block_scale_code(amax_b: float, s_t: float, flags: int = SCALE_ROUND_UP) -> int:
    return _load().oracle_e4m3_block_scale_code(float(amax_b), float(s_t), int(flags))


def e2m1_code(w: float, S: float) -> int:
    return _load().oracle_e2m1_code(float(w), float(S))


# -------------------------------------------------------------- quantizer --
def nvfp4_quantize(w_bits, flags: int = SCALE_ROUND_UP, tensor_scale_in: float | None = None,
                   threads: int = 0, stochastic_seed: int | None = None):
    """BF16 [N, K] bit patterns -> (packed u8 [N, K/2], scales u8 [N, K/16], s_t float32).
    stochastic_seed: stochastic element rounding with that seed (else nearest-even)."""
    w = _bits16(w_bits)
    if w.ndim != 2:
        raise ValueError("w must be 2-D")
    n, k = w.shape
    ldw = w.strides[0] // 2
    if w.strides[1] != 2:
        w = np.ascontiguousarray(w)
        ldw = k
    packed = np.zeros((n, k // 2), dtype=np.uint8)
    scales = np.zeros((n, k // 16), dtype=np.uint8)
    s_out = np.zeros(1, dtype=np.float32)
    s_in = None if tensor_scale_in is None else np.array([tensor_scale_in], dtype=np.float32)
    if stochastic_seed is None:
        rc = _load().oracle_nvfp4_quantize(_ptr(w), n, k, ldw, None if s_in is None else _ptr(s_in),
                                           int(flags), _ptr(packed), _ptr(scales), _ptr(s_out),
                                           int(threads))
    else:
        rc = _load().oracle_nvfp4_quantize_sr(_ptr(w), n, k, ldw, None if s_in is None else _ptr(s_in),
                                              int(flags), int(stochastic_seed) & (2 ** 64 - 1), _ptr(packed),
                                              _ptr(scales), _ptr(s_out), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_nvfp4_quantize rejected its arguments (rc={rc})")
    return packed, scales, np.float32(s_out[0])


def sr_uniform(seed: int, e: int) -> float:
    """The uniform in [0, 1) that stochastic rounding draws for element e."""
    return float(_load().oracle_sr_uniform(int(seed) & (2 ** 64 - 1), int(e)))


def e2m1_sr_mag(aw: float, S: float, u: float) -> int:
    return int(_load().oracle_e2m1_sr_mag(float(aw), float(S), float(u)))


def mxfp4_quantize(w_bits):
    """BF16 [N, K] bit patterns (K % 32 == 0) -> (packed u8 [N, K/2], E8M0 scales u8 [N, K/32])."""
    w = np.ascontiguousarray(_bits16(w_bits))
    n, k = w.shape
    packed = np.zeros((n, k // 2), dtype=np.uint8)
    scales = np.zeros((n, k // 32), dtype=np.uint8)
    rc = _load().oracle_mxfp4_quantize(_ptr(w), n, k, k, _ptr(packed), _ptr(scales))
    if rc != 0:
        raise ValueError(f"oracle_mxfp4_quantize rejected its arguments (rc={rc})")
    return packed, scales


def bf16_nearest_even(v: float) -> int:
    """Bit pattern of the BF16 value nearest to v (ties to the even code)."""
    return int(_load().oracle_bf16_nearest_even(float(v)))


def nvfp4_dequantize(packed, scales, s_t):
    """(fp64 [N, K] exact values, uint16 [N, K] BF16 bit patterns) of an NVFP4
    tensor: e2m1 x e4m3 x s_t, rounded once to the nearest BF16 (ties even)."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    n, k = packed.shape[0], packed.shape[1] * 2
    if scales.shape != (n, k // 16):
        raise ValueError(f"scales shape {scales.shape} != {(n, k // 16)}")
    f64 = np.zeros((n, k), dtype=np.float64)
    bits = np.zeros((n, k), dtype=np.uint16)
    rc = _load().oracle_nvfp4_dequantize(_ptr(packed), _ptr(scales), float(np.float32(s_t)), n, k, _ptr(f64),
                                         _ptr(bits))
    if rc != 0:
        raise ValueError(f"oracle_nvfp4_dequantize rejected its arguments (rc={rc})")
    return f64, bits


# ------------------------------------------------------------ W4A16 GEMM --
def w4a16_lora_gemm(x_bits, packed, scales, s_t, lora_a_bits=None, lora_b_bits=None,
                    lora_scale: float = 0.0, rows=None, threads: int = 0, x_f64=None) -> np.ndarray:
    """fp64 y[rows, N] = x w^T + lora_scale (x A^T) B^T with w dequantized exactly.
    x is BF16 bits, or (x_bits None) the fp64 activations x_f64."""
    if x_bits is None:
        x = np.ascontiguousarray(np.asarray(x_f64, dtype=np.float64))
    else:
        x = np.ascontiguousarray(_bits16(x_bits))
    m, k = x.shape
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    n = packed.shape[0]
    if packed.shape != (n, k // 2) or scales.shape != (n, k // 16):
        raise ValueError("packed/scales shape does not match x")
    r = 0
    a = b = None
    if lora_a_bits is not None:
        a = np.ascontiguousarray(_bits16(lora_a_bits))
        b = np.ascontiguousarray(_bits16(lora_b_bits))
        r = a.shape[0]
        if a.shape != (r, k) or b.shape != (n, r):
            raise ValueError("LoRA shapes must be A [r, K] and B [N, r]")
    rows_arr = None
    nrows = m
    if rows is not None:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.shape[0]
    y = np.zeros((nrows, n), dtype=np.float64)
    fn = _load().oracle_w4a16_lora_gemm if x_bits is not None else _load().oracle_w4a16_lora_gemm_f64
    rc = fn(
        _ptr(x), m, k, k, _ptr(packed), _ptr(scales), float(s_t), n,
        None if a is None else _ptr(a), None if b is None else _ptr(b), r, float(lora_scale),
        None if rows_arr is None else _ptr(rows_arr), nrows, _ptr(y), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_w4a16_lora_gemm rejected its arguments (rc={rc})")
    return y


# -------------------------------------------------------------------- AQN --
def aqn_sigma(stage: int, num_stages: int, sigma_start: float, sigma_end: float) -> float:
    return _load().oracle_aqn_sigma(int(stage), int(num_stages), float(sigma_start),
                                    float(sigma_end))


def philox4x64_10(counter, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint64).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint64).reshape(2))
    out = np.zeros(4, dtype=np.uint64)
    _load().oracle_philox4x64_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def aqn_noise(seed: int, step: int, layer: int, h: int) -> np.ndarray:
    z = np.zeros(h, dtype=np.float64)
    _load().oracle_aqn_noise(int(seed), int(step), int(layer), int(h), _ptr(z))
    return z


def rmsnorm(x_bits, w_eff, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(_bits16(x_bits))
    m, h = x.shape
    w = np.ascontiguousarray(np.asarray(w_eff, dtype=np.float64))
    y = np.zeros((m, h), dtype=np.float64)
    rc = _load().oracle_rmsnorm(_ptr(x), m, h, h, _ptr(w), float(eps), _ptr(y))
    if rc != 0:
        raise ValueError("oracle_rmsnorm rejected its arguments")
    return y


def w4a16_lora_backward(dy_bits, x_bits, packed, scales, s_t, lora_a_bits=None, lora_b_bits=None,
                        lora_scale: float = 0.0, threads: int = 0):
    """fp64 (dx [M, K], dA [r, K] or None, dB [N, r] or None) of the layer for upstream dy [M, N].
    threads: worker threads over independent output rows (0: one per core)."""
    dy = np.ascontiguousarray(_bits16(dy_bits))
    x = np.ascontiguousarray(_bits16(x_bits))
    m, n = dy.shape
    k = x.shape[1]
    if x.shape[0] != m or packed.shape != (n, k // 2) or scales.shape != (n, k // 16):
        raise ValueError("shapes do not match")
    r = 0
    a = b = None
    if lora_a_bits is not None:
        a = np.ascontiguousarray(_bits16(lora_a_bits))
        b = np.ascontiguousarray(_bits16(lora_b_bits))
        r = a.shape[0]
    dx = np.zeros((m, k))
    da = np.zeros((r, k)) if r else None
    db = np.zeros((n, r)) if r else None
    rc = _load().oracle_w4a16_lora_backward(
        _ptr(dy), _ptr(x), m, n, k, _ptr(np.ascontiguousarray(packed)), _ptr(np.ascontiguousarray(scales)),
        float(s_t), None if a is None else _ptr(a), None if b is None else _ptr(b), r, float(lora_scale),
        _ptr(dx), None if da is None else _ptr(da), None if db is None else _ptr(db), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_w4a16_lora_backward rejected its arguments (rc={rc})")
    return dx, da, db


def rmsnorm_w4a16_lora_gemm(x_bits, norm_weight, eps: float, packed, scales, s_t, lora_a_bits=None,
                            lora_b_bits=None, lora_scale: float = 0.0, rows=None, threads: int = 0) -> np.ndarray:
    """fp64 y = W4A16+LoRA layer of RMSNorm(x) with scale vector norm_weight:
    the norm's fp64 output, unrounded, is the layer's input."""
    xn = rmsnorm(x_bits, norm_weight, eps)
    return w4a16_lora_gemm(None, packed, scales, s_t, lora_a_bits, lora_b_bits, lora_scale, rows=rows,
                           threads=threads, x_f64=xn)


def aqn_rmsnorm(x_bits, weight, eps: float, sigma: float, seed: int, step: int, layer: int):
    """fp64 (y [M, H], noisy weight [H]) of RMSNorm with w + sigma z as its scale."""
    x = np.ascontiguousarray(_bits16(x_bits))
    m, h = x.shape
    w = np.ascontiguousarray(np.asarray(weight, dtype=np.float32))
    y = np.zeros((m, h), dtype=np.float64)
    wn = np.zeros(h, dtype=np.float64)
    rc = _load().oracle_aqn_rmsnorm(_ptr(x), m, h, h, _ptr(w), float(eps), float(sigma),
                                    int(seed), int(step), int(layer), _ptr(y), _ptr(wn))
    if rc != 0:
        raise ValueError("oracle_aqn_rmsnorm rejected its arguments")
    return y, wn
