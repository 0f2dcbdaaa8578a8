"""GPU qerl_w4a16_lora_backward against the fp64 oracle backward.

dx (BF16 output of an FP32 sum over N and the ranks) is held to the GEMM
tolerance (relative L2 <= 5e-3, max |err| <= 1e-2 max |ref|); dA and dB (FP32
sums of exact BF16 products, no output rounding) to relative L2 <= 1e-4 and
max |err| <= 1e-3 max |ref|."""
import numpy as np
import pytest
import torch

import nvfp4_weight_only_quantize_amd as q
import oracle
from nvfp4_weight_only_quantize_amd import synth
from parity import assert_gemm_close, bf16_to_f64, bits_to_gpu, dev, gemm_errors

pytestmark = pytest.mark.gpu


def _case(m, n, k, r, seed):
    w = synth.weight_bf16(n, k, seed=seed, row_lognormal_sigma=0.5)
    packed, scales, s_t = oracle.nvfp4_quantize(synth.bf16_bits(w), threads=16)
    x = synth.bf16_bits(synth.activation_bf16(m, k, seed=seed + 1, outlier_col_frac=0.01))
    dy = synth.bf16_bits(synth.activation_bf16(m, n, seed=seed + 2))
    a = b = None
    if r:
        a, b = synth.lora_bf16(n, k, r, seed=seed + 3)
        a, b = synth.bf16_bits(a), synth.bf16_bits(b)
    wq = q.NVFP4Weight(torch.from_numpy(packed).to(dev()), torch.from_numpy(scales).to(dev()),
                       torch.tensor([s_t], dtype=torch.float32, device=dev()))
    return dy, x, packed, scales, s_t, a, b, wq


def _check(m, n, k, r, seed, lam=2.0, strided=False, s_t_override=None):
    dy, x, packed, scales, s_t, a, b, wq = _case(m, n, k, r, seed)
    if s_t_override is not None:  # the same codes under another tensor scale
        s_t = np.float32(s_t_override)
        wq = q.NVFP4Weight(wq.packed, wq.scales, torch.tensor([s_t], dtype=torch.float32, device=dev()))
    dyg, xg = bits_to_gpu(dy), bits_to_gpu(x)
    if strided:
        big = torch.zeros((m, n + 24), dtype=torch.bfloat16, device=dev())
        big[:, :n] = dyg
        dyg = big[:, :n]
        bigx = torch.zeros((m, k + 40), dtype=torch.bfloat16, device=dev())
        bigx[:, :k] = xg
        xg = bigx[:, :k]
    ag = None if a is None else bits_to_gpu(a)
    bg = None if b is None else bits_to_gpu(b)
    dx, da, db = q.w4a16_lora_backward(dyg, xg, wq, ag, bg, lam)
    torch.cuda.synchronize()
    rdx, rda, rdb = oracle.w4a16_lora_backward(dy, x, packed, scales, s_t, a, b, lam, threads=16)
    what = f"m={m} n={n} k={k} r={r}"
    assert_gemm_close(bf16_to_f64(dx), rdx, "dx " + what)
    if r:
        for got, ref, nm in ((da, rda, "dA"), (db, rdb, "dB")):
            g = got.cpu().numpy().astype(np.float64)
            rel, mx = gemm_errors(g, ref)
            assert rel <= 1e-4 and mx <= 1e-3, f"{nm} {what}: rel_l2={rel:.3e} max={mx:.3e}"
    else:
        assert da is None and db is None


@pytest.mark.parametrize("mnkr", [(1, 16, 32, 4), (5, 40, 64, 8), (64, 96, 256, 16), (100, 130, 528, 32),
                                  (3, 33, 80, 0), (17, 256, 1024, 128), (128, 512, 1024, 32), (65, 64, 144, 24),
                                  (9, 37, 96, 5), (33, 2050, 2064, 3)])
def test_backward_small(mnkr):
    m, n, k, r = mnkr
    _check(m, n, k, r, seed=5000 + m + n + k + r)


def test_backward_strided_inputs():
    _check(40, 72, 256, 16, seed=5100, strided=True)


@pytest.mark.parametrize("proj", ["q", "k"])
def test_backward_7b_projection(proj):
    n, k = synth.QWEN25_7B[proj]
    _check(64, n, k, 32, seed=5200 + n)


@pytest.mark.parametrize("proj", ["q", "k", "gate", "down"])
def test_backward_7b_bench_shapes(proj):
    # the backward leg's shapes (M = 2048 tokens, r = 32), dx, dA and dB in
    # full: 16 row blocks of dx, four M chunks of the rank products, and the
    # widest N (gate, 18944) and K (down, 18944) of the layer
    n, k = synth.QWEN25_7B[proj]
    _check(2048, n, k, 32, seed=5300 + n + k)


def test_backward_many_m_chunks_ragged():
    # m = 1100: three M chunks of the rank products (the last one partial) and
    # nine dx row blocks, the last one ragged (7B k/v projection)
    n, k = synth.QWEN25_7B["k"]
    _check(1100, n, k, 32, seed=5400)


def test_backward_rejects_non_contiguous_lora():
    n, k, r, m = 64, 256, 16, 8
    dy, x, packed, scales, s_t, a, b, wq = _case(m, n, k, r, seed=5500)
    ag, bg = bits_to_gpu(a), bits_to_gpu(b)
    a_view = ag.t().contiguous().t()  # [r, k] with strides (1, r)
    b_view = bg.t().contiguous().t()
    with pytest.raises(ValueError):
        q.w4a16_lora_backward(bits_to_gpu(dy), bits_to_gpu(x), wq, a_view, bg, 2.0)
    with pytest.raises(ValueError):
        q.w4a16_lora_backward(bits_to_gpu(dy), bits_to_gpu(x), wq, ag, b_view, 2.0)


@pytest.mark.parametrize("s_t", [1e-39, 1e-30, 1e-18])
def test_backward_tiny_tensor_scale(s_t):
    """lambda / s_t overflows FP32 (1e-39, a subnormal) or exceeds the folding
    bound (1e-30): the LoRA term is added outside the accumulation; 1e-18
    still folds.  dx is then dominated by the LoRA term."""
    _check(100, 130, 528, 32, seed=5300, s_t_override=s_t)
    _check(70, 64, 144, 8, seed=5301, s_t_override=s_t)
