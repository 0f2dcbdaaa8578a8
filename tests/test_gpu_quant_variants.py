"""GPU quantizer variants against the oracle, bit for bit:
qerl_nvfp4_quantize_stochastic (stochastic element rounding, same block
scales as the deterministic quantizer) and qerl_mxfp4_quantize (OCP MX:
E2M1 codes, one E8M0 scale per 32 elements)."""
import numpy as np
import pytest
import torch

import nvfp4_weight_only_quantize_amd as q
import oracle
from nvfp4_weight_only_quantize_amd import synth
from parity import bits_to_gpu, dev
from test_gpu_quantize import _dist

pytestmark = pytest.mark.gpu


def _sr_compare(bits, seed, flags=0, s_in=None, w_gpu=None):
    if w_gpu is None:
        w_gpu = bits_to_gpu(bits)
    s_in_t = None if s_in is None else torch.tensor([s_in], dtype=torch.float32, device=dev())
    r = q.nvfp4_quantize(w_gpu, flags=flags, tensor_scale_in=s_in_t, check_finite=False, stochastic_seed=seed)
    torch.cuda.synchronize()
    gp, gs, gt = r.packed.cpu().numpy(), r.scales.cpu().numpy(), np.float32(r.tensor_scale.cpu().numpy()[0])
    op, os_, ot = oracle.nvfp4_quantize(bits, flags=flags, tensor_scale_in=s_in, threads=16, stochastic_seed=seed)
    assert gt.view(np.uint32) == np.float32(ot).view(np.uint32)
    assert np.array_equal(gs, os_)
    bad = np.argwhere(gp != op)
    assert bad.size == 0, f"packed bytes differ at {bad[:5].tolist()}"
    return gp


KINDS = ["normal", "rowscale", "wide", "tiny_blocks", "heavy", "tiny_tensor", "subnormal_scale"]


@pytest.mark.parametrize("shape", [(1, 16), (7, 48), (64, 512), (130, 1040)])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("flags", [0, 1])
def test_stochastic_bit_exact(shape, kind, flags):
    bits = _dist(kind, *shape, seed=shape[0] * 31 + shape[1] + KINDS.index(kind))
    _sr_compare(bits, seed=4242 + shape[0], flags=flags)


def test_stochastic_seeds_differ_and_repeat():
    bits = _dist("normal", 64, 512, seed=3)
    a = _sr_compare(bits, seed=1)
    b = _sr_compare(bits, seed=2)
    assert not np.array_equal(a, b)
    assert np.array_equal(a, _sr_compare(bits, seed=1))
    _sr_compare(bits, seed=2 ** 64 - 1)


def test_stochastic_strided_and_supplied_scale():
    bits = _dist("heavy", 40, 256, seed=4)
    full = np.zeros((40, 320), dtype=np.uint16)
    full[:, :256] = bits
    w = bits_to_gpu(full)[:, :256]
    _sr_compare(bits, seed=9, w_gpu=w)
    _sr_compare(bits, seed=9, s_in=1e-3)
    _sr_compare(bits, seed=9, s_in=2.0 ** -100)  # tiny tensor scale


def test_stochastic_7b_projection():
    n, k = synth.QWEN25_7B["q"]
    bits = synth.bf16_bits(synth.weight_bf16(n, k, seed=77, row_lognormal_sigma=0.5))
    _sr_compare(bits, seed=1002)


def _mx_compare(bits, w_gpu=None):
    if w_gpu is None:
        w_gpu = bits_to_gpu(bits)
    gp, gs = q.mxfp4_quantize(w_gpu)
    torch.cuda.synchronize()
    gp, gs = gp.cpu().numpy(), gs.cpu().numpy()
    op, os_ = oracle.mxfp4_quantize(bits)
    assert np.array_equal(gs, os_), np.argwhere(gs != os_)[:5].tolist()
    ok_rows = gs != 0xFF  # a non-finite block's codes are unspecified
    okp = np.repeat(ok_rows, 16, axis=1)
    bad = np.argwhere((gp != op) & okp)
    assert bad.size == 0, f"packed bytes differ at {bad[:5].tolist()}"


@pytest.mark.parametrize("shape", [(1, 32), (7, 64), (64, 512), (130, 1056)])
@pytest.mark.parametrize("kind", KINDS)
def test_mxfp4_bit_exact(shape, kind):
    _mx_compare(_dist(kind, *shape, seed=shape[0] * 37 + shape[1] + KINDS.index(kind)))


def test_mxfp4_special_blocks():
    k = 256
    vals = np.random.default_rng(8).standard_normal((4, k)).astype(np.float32)
    vals[0, :32] = 0.0                      # all-zero block
    vals[0, 32:64] = -0.0                   # negative zeros
    vals[1, :32] *= 2.0 ** -130             # subnormal BF16 amax
    vals[1, 32:64] = 6.0 * 2.0 ** 20        # amax on a power-of-two boundary
    vals[2, 64] = np.inf                    # non-finite blocks
    vals[2, 100] = np.nan
    vals[3, :] *= 2.0 ** 120                # near the top of the range
    bits = synth.bf16_bits(torch.from_numpy(vals).to(torch.bfloat16))
    _mx_compare(bits)
    gs = q.mxfp4_quantize(bits_to_gpu(bits))[1].cpu().numpy()
    assert gs[0, 0] == 0 and gs[2, 2] == 0xFF and gs[2, 3] == 0xFF


def test_mxfp4_strided_and_7b_projection():
    bits = _dist("normal", 40, 256, seed=5)
    full = np.zeros((40, 320), dtype=np.uint16)
    full[:, :256] = bits
    _mx_compare(bits, w_gpu=bits_to_gpu(full)[:, :256])
    n, k = synth.QWEN25_7B["gate"]
    _mx_compare(synth.bf16_bits(synth.weight_bf16(n, k, seed=78, row_lognormal_sigma=0.5)))
