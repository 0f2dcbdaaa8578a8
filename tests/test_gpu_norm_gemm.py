"""GPU qerl_rmsnorm_w4a16_lora_gemm_multi (RMSNorm + projections in one call)
and qerl_aqn_noisy_weight.

The fused path (M <= 16, K % 32 == 0) and the two-launch path (a norm launch,
then the projections) are both compared with the fp64 oracle composite: the
oracle's RMSNorm output, unrounded, fed to the oracle layer, with the same
FP32 scale vector (the AQN noisy weight, drawn by the oracle).  Tolerances are
the GEMM's (relative L2 <= 5e-3, max |y - y_ref| <= 1e-2 max |y_ref|); the
noisy weight is held to the AQN FP32 bound (1e-5 relative) and to bit
equality with what qerl_aqn_rmsnorm multiplies by.
"""
import numpy as np
import pytest
import torch

import nvfp4_weight_only_quantize_amd as q
import oracle
from nvfp4_weight_only_quantize_amd import synth
from parity import AQN_REL, assert_gemm_close, bf16_to_f64, bits_to_gpu, dev, gemm_errors
from test_gpu_gemm import Layer, _x

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _noisy(k, seed, sigma=2e-2, step=3, layer=5):
    """The oracle's noisy norm weight, as the FP32 vector both sides use."""
    w = (1.0 + 0.1 * np.random.default_rng(seed).standard_normal(k)).astype(np.float32)
    x1 = np.zeros((1, k), dtype=np.uint16)
    _, wn = oracle.aqn_rmsnorm(x1 | 0x3F80, w, EPS, sigma, seed, step, layer)
    return w, wn.astype(np.float32)


def _check(layers, m, k, seed, rows=None):
    x = _x(m, k, seed=seed, outliers=0.01)
    _, wn = _noisy(k, seed + 1)
    xg = bits_to_gpu(x)
    wg = torch.from_numpy(wn).to(dev())
    outs = q.rmsnorm_w4a16_lora_gemm_multi(xg, wg, EPS, [(L.wq, L.a, L.b, L.lam) for L in layers])
    torch.cuda.synchronize()
    for i, (L, y) in enumerate(zip(layers, outs)):
        y = bf16_to_f64(y)
        ref = oracle.rmsnorm_w4a16_lora_gemm(x, wn, EPS, L.packed, L.scales, L.s_t, L.a_bits, L.b_bits, L.lam,
                                             rows=rows, threads=16)
        assert_gemm_close(y if rows is None else y[rows], ref, f"segment {i} n={L.n} r={L.r} m={m} k={k}")


@pytest.mark.parametrize("m", [1, 8, 16, 24, 64])
def test_norm_7b_qkv(m):
    k = synth.QWEN25_7B["q"][1]
    layers = [Layer(synth.QWEN25_7B[p][0], k, 32, seed=synth.seed_for(1016, p)) for p in ("q", "k", "v")]
    _check(layers, m, k, seed=synth.seed_for(1016, "x", m), rows=None if m <= 8 else [0, 5, m - 1])


@pytest.mark.parametrize("m", [1, 16])
def test_norm_7b_gate_up(m):
    n, k = synth.QWEN25_7B["gate"]
    layers = [Layer(n, k, 32, seed=synth.seed_for(1017, p)) for p in ("gate", "up")]
    _check(layers, m, k, seed=synth.seed_for(1017, "x", m), rows=None if m == 1 else [0, 9, 15])


@pytest.mark.parametrize("m", [1, 3, 5, 16, 17, 40, 100])
def test_norm_mixed_ranks_and_widths(m):
    # ranks 16, 0, 8, 4 and widths off the unit; m = 17 .. 64 and m > 64 take
    # the norm launch + projections
    k = 512
    layers = [Layer(n, k, r, seed=2100 + n + r) for n, r in ((96, 16), (77, 0), (130, 8), (64, 4))]
    _check(layers, m, k, seed=2200 + m)


@pytest.mark.parametrize("m,k", [(1, 528), (4, 528), (2, 1040)])
def test_norm_k_not_multiple_of_32(m, k):
    # k % 32 != 0: the norm launch + projections path
    layers = [Layer(n, k, r, seed=2300 + n + k) for n, r in ((64, 8), (33, 0))]
    _check(layers, m, k, seed=2400 + m + k)


@pytest.mark.parametrize("m,r", [(1, 0), (8, 0), (2, 128), (16, 128)])
def test_norm_single_segment_rank_ends(m, r):
    # no LoRA (producers only sum squares) and the largest rank
    k = 1024
    _check([Layer(200, k, r, seed=2500 + r)], m, k, seed=2600 + m + r)


def test_norm_fused_matches_two_launches():
    # the fused launch against the standalone norm (BF16 rows) + projections
    k = 3584
    layers = [Layer(synth.QWEN25_7B[p][0], k, 32, seed=synth.seed_for(1018, p)) for p in ("q", "k", "v")]
    for m in (1, 8, 16):
        x = _x(m, k, seed=2700 + m, outliers=0.01)
        w, _ = _noisy(k, 2800 + m)
        xg = bits_to_gpu(x)
        wn = q.aqn_noisy_weight(torch.from_numpy(w).to(dev()), 2e-2, seed=7, step=1, layer_id=2)
        fused = q.rmsnorm_w4a16_lora_gemm_multi(xg, wn, EPS, [(L.wq, L.a, L.b, L.lam) for L in layers])
        _, xn = q.aqn_rmsnorm(xg, torch.from_numpy(w).to(dev()), EPS, 2e-2, seed=7, step=1, layer_id=2,
                              want_f32=False, want_bf16=True)
        plain = q.w4a16_lora_gemm_multi(xn, [(L.wq, L.a, L.b, L.lam) for L in layers])
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(fused, plain)):
            rel, mx = gemm_errors(bf16_to_f64(a), bf16_to_f64(b))
            assert rel <= 5e-3 and mx <= 1e-2, f"m={m} segment {i}: rel_l2={rel:.3e} max={mx:.3e}"


def test_noisy_weight_matches_oracle_and_the_norm():
    h = 3584
    w = (1.0 + 0.1 * np.random.default_rng(11).standard_normal(h)).astype(np.float32)
    wg = torch.from_numpy(w).to(dev())
    for sigma, seed, step, layer in ((1e-2, 1, 0, 0), (5e-2, 2 ** 40 + 3, 7, 27), (0.0, 5, 1, 1)):
        got = q.aqn_noisy_weight(wg, sigma, seed=seed, step=step, layer_id=layer)
        x1 = np.full((1, h), 0x3F80, dtype=np.uint16)
        _, ref = oracle.aqn_rmsnorm(x1, w, EPS, sigma, seed, step, layer)
        g = got.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(g - ref) <= AQN_REL * np.maximum(np.abs(ref), 1e-30)), (sigma, seed)
        wn = torch.empty(h, dtype=torch.float32, device=dev())
        q.aqn_rmsnorm(bits_to_gpu(x1), wg, EPS, sigma, seed=seed, step=step, layer_id=layer, noisy_weight_out=wn)
        torch.cuda.synchronize()
        assert torch.equal(got, wn)
    # in place (out is weight)
    v = wg.clone()
    q.aqn_noisy_weight(v, 1e-2, seed=1, out=v)
    assert torch.equal(v, q.aqn_noisy_weight(wg, 1e-2, seed=1))


def test_norm_shared_workspace_is_repeatable():
    # fused-norm calls, plain multi calls and single calls of several shapes on
    # one workspace (any contents): every repeat is bit-identical
    k = 3584
    qkv = [Layer(synth.QWEN25_7B[p][0], k, 32, seed=synth.seed_for(1019, p)) for p in ("q", "k", "v")]
    gu = [Layer(synth.QWEN25_7B[p][0], k, 32, seed=synth.seed_for(1019, p)) for p in ("gate", "up")]
    cases = [(1, qkv), (8, gu), (16, qkv), (24, gu), (3, gu)]
    need = max(max(q.rmsnorm_w4a16_lora_gemm_multi_workspace_size(m, k, [(L.n, L.r) for L in ls]),
                   q.w4a16_lora_gemm_multi_workspace_size(m, k, [(L.n, L.r) for L in ls])) for m, ls in cases)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=dev())  # any contents
    _, wn = _noisy(k, 2900)
    wg = torch.from_numpy(wn).to(dev())
    xs = {m: bits_to_gpu(_x(m, k, seed=3000 + m)) for m, _ in cases}
    first = None
    for rep in range(3):
        got = []
        for m, ls in cases:
            segs = [(L.wq, L.a, L.b, L.lam) for L in ls]
            got.append(q.rmsnorm_w4a16_lora_gemm_multi(xs[m], wg, EPS, segs, workspace=ws))
            got.append(q.w4a16_lora_gemm_multi(xs[m], segs, workspace=ws))
        torch.cuda.synchronize()
        if first is None:
            first = [[y.clone() for y in g] for g in got]
        else:
            for a, b in zip(first, got):
                for ya, yb in zip(a, b):
                    assert torch.equal(ya, yb)
