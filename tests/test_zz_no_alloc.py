"""qerl_w4a16_lora_gemm_noalloc (static per-device scratch, no workspace
argument) against qerl_w4a16_lora_gemm with its own workspace: the same
kernels on the same inputs, so the outputs must be bit-identical.  The calls
run back to back on one stream, each later one smaller than the one before,
so a later call runs on the scratch the earlier one left behind."""
import pytest
import torch

import nvfp4_weight_only_quantize_amd as q
from nvfp4_weight_only_quantize_amd import synth
from parity import dev

pytestmark = pytest.mark.gpu


def _case(m, n, k, r, seed):
    w = synth.weight_bf16(n, k, seed=seed, row_lognormal_sigma=0.5, device=dev())
    wq = q.nvfp4_quantize(w)
    a, b = synth.lora_bf16(n, k, r, seed=seed + 1, device=dev()) if r else (None, None)
    x = synth.activation_bf16(m, k, seed=seed + 2, outlier_col_frac=0.005, device=dev())
    return x, wq, a, b


# (m, n, k, r): the 32B gate at m = 64 (35 MB of scratch, MFMA decode route),
# a ragged prefill-route shape (split-K partials), the 7B down at m = 8
# (stream route, K = 18944), the 7B q at m = 1, and a tiny ragged one
SEQUENCE = [(64, 27648, 5120, 32), (300, 1000, 2048, 16), (8, 3584, 18944, 32), (1, 3584, 3584, 32),
            (3, 77, 512, 8)]


def test_noalloc_matches_workspace_call():
    prev = None
    for i, (m, n, k, r) in enumerate(SEQUENCE):
        need = q.w4a16_lora_gemm_workspace_size(m, n, k, r)
        assert need <= q.NOALLOC_SCRATCH_BYTES
        if prev is not None:
            assert need < prev, "each call must be smaller than the one before"
        prev = need
        print(f"noalloc case {i}: m={m} n={n} k={k} r={r} scratch {need} B", flush=True)
        x, wq, a, b = _case(m, n, k, r, seed=7000 + 13 * i)
        lam = 2.0
        y_ws = q.w4a16_lora_gemm(x, wq, a, b, lam)
        y_na = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=dev())
        q.w4a16_lora_gemm_noalloc(x, wq, a, b, lam, out=y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), f"case {i} differs"
        # the same call again on the scratch it just left: same bits
        q.w4a16_lora_gemm_noalloc(x, wq, a, b, lam, out=y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), f"case {i} repeat differs"


def test_noalloc_under_graph_capture():
    m, n, k, r = 16, 4096, 3584, 32
    x, wq, a, b = _case(m, n, k, r, seed=7100)
    y_ws = q.w4a16_lora_gemm(x, wq, a, b, 2.0)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q.w4a16_lora_gemm_noalloc(x, wq, a, b, 2.0, out=y)  # first call on the device outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.w4a16_lora_gemm_noalloc(x, wq, a, b, 2.0, out=y)
    for rep in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ws.view(torch.int16)), f"replay {rep} differs"
        # eager work on the shared scratch between replays
        q.w4a16_lora_gemm_noalloc(x[:1], wq, a, b, 2.0, out=torch.empty((1, n), dtype=torch.bfloat16,
                                                                          device=dev()))
        torch.cuda.synchronize()
    del g


def test_noalloc_rejects_sizes_above_the_scratch():
    m, n, k, r = 128, 27648, 5120, 32  # needs about 69 MB of partial sums
    assert q.w4a16_lora_gemm_workspace_size(m, n, k, r) > q.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((m, k), dtype=torch.bfloat16, device=dev())
    wq = q.NVFP4Weight(torch.zeros((n, k // 2), dtype=torch.uint8, device=dev()),
                       torch.zeros((n, k // 16), dtype=torch.uint8, device=dev()),
                       torch.ones(1, dtype=torch.float32, device=dev()))
    a = torch.zeros((r, k), dtype=torch.bfloat16, device=dev())
    b = torch.zeros((n, r), dtype=torch.bfloat16, device=dev())
    y = torch.full((m, n), 3.0, dtype=torch.bfloat16, device=dev())
    with pytest.raises(q.QerlError, match="scratch"):
        q.w4a16_lora_gemm_noalloc(x, wq, a, b, 1.0, out=y)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()), "a rejected call must not write its output"
