"""GPU quantizer (qerl_nvfp4_quantize) against the oracle: bit-exact packed
codes, scale bytes and tensor scale."""
import numpy as np
import pytest
import torch

import oracle
import nvfp4_weight_only_quantize_amd as q
from nvfp4_weight_only_quantize_amd import synth
from golden_tables import E2M1, E4M3, f64_to_bf16_bits_exact
from parity import bits_to_gpu, dev

pytestmark = pytest.mark.gpu


def _gpu_quant(w_gpu, flags=0, s_in=None):
    s_in_t = None if s_in is None else torch.tensor([s_in], dtype=torch.float32, device=dev())
    r = q.nvfp4_quantize(w_gpu, flags=flags, tensor_scale_in=s_in_t, check_finite=False)
    torch.cuda.synchronize()
    return r.packed.cpu().numpy(), r.scales.cpu().numpy(), np.float32(r.tensor_scale.cpu().numpy()[0])


def _compare(bits, flags=0, s_in=None, w_gpu=None, threads=0):
    if w_gpu is None:
        w_gpu = bits_to_gpu(bits)
    gp, gs, gt = _gpu_quant(w_gpu, flags, s_in)
    op, os_, ot = oracle.nvfp4_quantize(bits, flags=flags, tensor_scale_in=s_in, threads=threads)
    if np.isnan(ot):
        assert np.isnan(gt)
        return
    assert gt.view(np.uint32) == np.float32(ot).view(np.uint32), (gt, ot)
    bad_s = np.argwhere(gs != os_)
    assert bad_s.size == 0, f"scale bytes differ at {bad_s[:5].tolist()}"
    bad_p = np.argwhere(gp != op)
    if bad_p.size:
        i = tuple(bad_p[0])
        raise AssertionError(f"packed bytes differ at {bad_p[:5].tolist()}: gpu={gp[i]:#x} oracle={op[i]:#x}")


def _dist(kind, n, k, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        v = rng.normal(0, 0.02, size=(n, k))
    elif kind == "rowscale":
        v = rng.normal(0, 0.02, size=(n, k)) * np.exp(rng.normal(0, 0.5, size=(n, 1)))
    elif kind == "wide":
        v = rng.normal(0, 1, size=(n, k)) * 2.0 ** rng.integers(-30, 30, size=(n, 1))
    elif kind == "tiny_blocks":
        v = rng.normal(0, 1, size=(n, k))
        v[:, ::3] *= 1e-9
    elif kind == "heavy":
        v = rng.standard_t(1.5, size=(n, k))
    elif kind == "tiny_tensor":     # s_t far below 2^-90: the double-precision path
        v = rng.normal(0, 1, size=(n, k)) * 2.0 ** -100
    elif kind == "subnormal_scale":  # s_t is an FP32 subnormal
        v = rng.normal(0, 1, size=(n, k)) * 2.0 ** -118
    else:
        raise ValueError(kind)
    return synth.bf16_bits(torch.tensor(v, dtype=torch.float64).to(torch.bfloat16))


SHAPES = [(1, 16), (3, 48), (17, 80), (64, 2048), (5, 4096), (130, 272)]
KINDS = ["normal", "rowscale", "wide", "tiny_blocks", "heavy", "tiny_tensor", "subnormal_scale"]


@pytest.mark.parametrize("flags", [q.SCALE_ROUND_UP, q.SCALE_RNE])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("shape", SHAPES)
def test_bit_exact_small(shape, kind, flags):
    n, k = shape
    bits = _dist(kind, n, k, seed=n * 131 + k + KINDS.index(kind))
    _compare(bits, flags)


@pytest.mark.parametrize("flags", [q.SCALE_ROUND_UP, q.SCALE_RNE])
def test_representable_round_trip(flags):
    rng = np.random.default_rng(5)
    n, k = 40, 256
    codes = rng.integers(0, 16, size=(n, k))
    codes[:, ::16] = 7
    scales = rng.integers(1, 0x7F, size=(n, k // 16))
    scales[3, 2] = 0x7E
    vals = np.array(E2M1)[codes] * np.repeat(E4M3[scales], 16, axis=1) * 2.0 ** -12
    bits = f64_to_bf16_bits_exact(vals)
    _compare(bits, flags)
    gp, gs, gt = _gpu_quant(bits_to_gpu(bits), flags)
    assert float(gt) == 2.0 ** -12
    assert np.array_equal(gs, scales.astype(np.uint8))
    assert np.array_equal(gp, (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))


def test_strided_rows():
    bits = _dist("rowscale", 33, 160, 7)
    wide = torch.zeros((33, 200), dtype=torch.bfloat16, device=dev())
    wide[:, :160] = bits_to_gpu(bits)
    _compare(bits, 0, w_gpu=wide[:, :160])


def test_zero_tensor_and_zero_blocks():
    bits = np.zeros((8, 64), dtype=np.uint16)
    bits[2, 5] = 0x8000
    _compare(bits)
    bits2 = _dist("normal", 8, 64, 9)
    bits2[3, 16:32] = 0
    bits2[4, 0:16] = 0x8000
    _compare(bits2)


@pytest.mark.parametrize("bad", [0x7F80, 0xFF80, 0x7FC1])
def test_non_finite_gives_nan_scale(bad):
    bits = _dist("normal", 16, 64, 11)
    bits[9, 33] = bad
    _, _, gt = _gpu_quant(bits_to_gpu(bits))
    assert np.isnan(gt)
    with pytest.raises(q.QerlError):
        q.nvfp4_quantize(bits_to_gpu(bits))


@pytest.mark.parametrize("s_in", [1e-5, 3.3e-4, 2.0 ** -20, 7.0])
def test_supplied_tensor_scale(s_in):
    bits = _dist("rowscale", 24, 320, 13)
    _compare(bits, 0, s_in=s_in)
    _compare(bits, 1, s_in=s_in)


@pytest.mark.parametrize("num,den", [(1, 3), (1, 7), (5, 21), (3, 7), (1, 21)])
def test_quotients_next_to_midpoints(num, den):
    """Elements +-n 2^j (n < 16) with s_t = fl(num / den): many |w| / (e s_t)
    land within 2^-24 of an E2M1 midpoint (e.g. 3 f / e = 0.75 for s_t ~ 1/3),
    where only the exact comparison decides the side."""
    rng = np.random.default_rng(100 * den + num)
    n = rng.integers(1, 16, size=(64, 256))
    j = rng.integers(-8, 2, size=(64, 256))
    sign = rng.choice([-1.0, 1.0], size=(64, 256))
    vals = (sign * n * np.exp2(j)).astype(np.float32)  # 4-bit significands: exact in BF16
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    s_in = float(np.float32(num / den))
    _compare(bits, 0, s_in=s_in)
    _compare(bits, 1, s_in=s_in)


def test_invalid_supplied_tensor_scale_gives_nan():
    bits = _dist("normal", 4, 32, 14)
    for s_in in (0.0, -1.0, float("inf"), float("nan")):
        _, _, gt = _gpu_quant(bits_to_gpu(bits), 0, s_in)
        assert np.isnan(gt)


def test_config1_layer():
    w = synth.weight_bf16(2048, 2048, seed=1001)
    _compare(synth.bf16_bits(w))


@pytest.mark.parametrize("name,shape", [("7b_down", (3584, 18944)), ("32b_gate", (27648, 5120))])
def test_full_size_tensor(name, shape):
    n, k = shape
    w = synth.weight_bf16(n, k, seed=2000 + n, row_lognormal_sigma=0.5)
    _compare(synth.bf16_bits(w), threads=16)


@pytest.mark.parametrize("proj", ["q", "k", "down"])
def test_whole_model_config_layer(proj):
    # 32B-shaped layer with 0.1 % outlier output rows x20 (the whole-model pass)
    n, k = synth.QWEN25_32B[proj]
    w = synth.weight_bf16(n, k, seed=synth.seed_for(1005, 17, proj), outlier_row_frac=0.001)
    _compare(synth.bf16_bits(w), threads=16)
