"""GPU qerl_nvfp4_dequantize against the oracle, bit for bit.

Random code and scale bytes (every E2M1 code; E4M3 bytes including the NaN
encodings) with tensor scales that exercise BF16 ties, subnormal results and
overflow to infinity; shapes with one block, ragged row counts and a padded
output stride; the quantizer's own output at a 7B projection's full size.
"""
import numpy as np
import pytest
import torch

import nvfp4_weight_only_quantize_amd as q
import oracle
from nvfp4_weight_only_quantize_amd import synth
from parity import dev

pytestmark = pytest.mark.gpu


def _weight(packed, scales, s_t):
    d = dev()
    return q.NVFP4Weight(torch.from_numpy(packed).to(d), torch.from_numpy(scales).to(d),
                         torch.tensor([s_t], dtype=torch.float32, device=d))


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n,k", [(1, 16), (5, 48), (130, 272), (64, 3584), (1000, 1040)])
@pytest.mark.parametrize("s_t", [1.0, 0.0123, 3.0e-41, 2.5e36, 7.7e-39])
def test_dequantize_bit_exact(n, k, s_t):
    rng = np.random.default_rng(n * 131 + k)
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (n, k // 16), dtype=np.uint8)
    _, ref = oracle.nvfp4_dequantize(packed, scales, np.float32(s_t))
    got = _bits(q.nvfp4_dequantize(_weight(packed, scales, np.float32(s_t))))
    nan_ref = (ref & 0x7FFF) > 0x7F80
    assert np.array_equal((got & 0x7FFF) > 0x7F80, nan_ref)
    np.testing.assert_array_equal(got[~nan_ref], ref[~nan_ref])


def test_dequantize_padded_stride_leaves_padding():
    n, k, ldo = 33, 160, 200
    rng = np.random.default_rng(3)
    packed = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (n, k // 16), dtype=np.uint8)
    big = torch.full((n, ldo), 7.0, dtype=torch.bfloat16, device=dev())
    q.nvfp4_dequantize(_weight(packed, scales, np.float32(0.37)), out=big[:, :k])
    _, ref = oracle.nvfp4_dequantize(packed, scales, np.float32(0.37))
    np.testing.assert_array_equal(_bits(big[:, :k].contiguous()), ref)
    assert bool((big[:, k:] == 7.0).all())


def test_dequantize_quantizer_output_7b_gate():
    # the quantizer's own output for the 7B gate projection, every element
    n, k = synth.QWEN25_7B["gate"]
    w = synth.weight_bf16(n, k, seed=synth.seed_for(1101, "gate"), row_lognormal_sigma=0.5, device=dev())
    wq = q.nvfp4_quantize(w)
    del w
    got = _bits(q.nvfp4_dequantize(wq))
    _, ref = oracle.nvfp4_dequantize(wq.packed.cpu().numpy(), wq.scales.cpu().numpy(),
                                     np.float32(wq.tensor_scale.item()))
    np.testing.assert_array_equal(got, ref)
