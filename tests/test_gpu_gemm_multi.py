"""GPU qerl_w4a16_lora_gemm_multi: several projections of one activation in
one call (for M <= 256 one launch), each against the fp64 oracle and against
the single-projection call; bit-for-bit repeatability with a shared workspace.
Tolerances as for the single call (relative L2 <= 5e-3, max |y - y_ref| <=
1e-2 max |y_ref|)."""
import pytest
import torch

import nvfp4_weight_only_quantize_amd as q
from nvfp4_weight_only_quantize_amd import synth
from parity import assert_gemm_close, bf16_to_f64, bits_to_gpu, dev
from test_gpu_gemm import Layer, _x

pytestmark = pytest.mark.gpu


def _check(layers, m, k, seed, rows=None):
    x = _x(m, k, seed=seed)
    xg = bits_to_gpu(x)
    outs = q.w4a16_lora_gemm_multi(xg, [(L.wq, L.a, L.b, L.lam) for L in layers])
    torch.cuda.synchronize()
    for i, (L, y) in enumerate(zip(layers, outs)):
        y = bf16_to_f64(y)
        ref = L.ref(x, rows=rows)
        assert_gemm_close(y if rows is None else y[rows], ref, f"segment {i} n={L.n} r={L.r} m={m}")
        single = bf16_to_f64(L.gpu(xg))
        assert_gemm_close(y, single, f"segment {i} against the single call, m={m}")


@pytest.mark.parametrize("m", [1, 8, 64, 128])
def test_multi_7b_qkv(m):
    k = synth.QWEN25_7B["q"][1]
    layers = [Layer(synth.QWEN25_7B[p][0], k, 32, seed=synth.seed_for(1006, p)) for p in ("q", "k", "v")]
    _check(layers, m, k, seed=synth.seed_for(1006, "x", m), rows=None if m <= 8 else [0, 9, 40, m - 1])


@pytest.mark.parametrize("m", [1, 16])
def test_multi_7b_gate_up(m):
    n, k = synth.QWEN25_7B["gate"]
    layers = [Layer(n, k, 32, seed=synth.seed_for(1007, p)) for p in ("gate", "up")]
    _check(layers, m, k, seed=synth.seed_for(1007, "x", m), rows=None if m == 1 else [0, 7, 15])


@pytest.mark.parametrize("m", [1, 5, 24, 100, 200, 257])
def test_multi_mixed_ranks_and_widths(m):
    # four segments: ranks 16, 0 (no LoRA), 8, 4 and widths that are no
    # multiple of the unit; m = 100 takes eight m-tiles per unit, m = 200 two
    # m-blocks of them, m = 257 the large-m path one segment at a time
    k = 512
    layers = [Layer(n, k, r, seed=1100 + n + r) for n, r in ((96, 16), (77, 0), (130, 8), (64, 4))]
    _check(layers, m, k, seed=1200 + m)


def test_multi_shared_workspace_is_repeatable():
    # one workspace (any contents) over a sequence of multi and single calls
    # of different shapes: every repeat is bit-identical to the first
    k = 3584
    qkv = [Layer(synth.QWEN25_7B[p][0], k, 32, seed=synth.seed_for(1008, p)) for p in ("q", "k", "v")]
    gu = [Layer(synth.QWEN25_7B[p][0], k, 32, seed=synth.seed_for(1008, p)) for p in ("gate", "up")]
    cases = [(1, qkv), (8, gu), (64, qkv), (3, gu)]
    need = max(max(q.w4a16_lora_gemm_multi_workspace_size(m, k, [(L.n, L.r) for L in ls]),
                   q.w4a16_lora_gemm_workspace_size(m, qkv[0].n, k, 32)) for m, ls in cases)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=dev())  # any contents
    xs = {m: bits_to_gpu(_x(m, k, seed=1300 + m)) for m, _ in cases}
    first = None
    for rep in range(3):
        got = []
        for m, ls in cases:
            got.append(q.w4a16_lora_gemm_multi(xs[m], [(L.wq, L.a, L.b, L.lam) for L in ls], workspace=ws))
            got.append([q.w4a16_lora_gemm(xs[m], qkv[0].wq, qkv[0].a, qkv[0].b, qkv[0].lam, workspace=ws)])
        torch.cuda.synchronize()
        if first is None:
            first = [[y.clone() for y in g] for g in got]
        else:
            for a, b in zip(first, got):
                for ya, yb in zip(a, b):
                    assert torch.equal(ya, yb)
