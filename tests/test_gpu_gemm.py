"""GPU W4A16 + LoRA layer (qerl_w4a16_lora_gemm) against the fp64 oracle.

The NVFP4 weights fed to the GPU are the oracle's own quantization, so this
file tests the GEMM independently of the GPU quantizer.  Tolerances: relative
L2 <= 5e-3 and max |y - y_ref| <= 1e-2 max |y_ref| (BF16 output rounding alone
gives ~1e-3 and ~4e-3)."""
import numpy as np
import pytest
import torch

import oracle
import nvfp4_weight_only_quantize_amd as q
from nvfp4_weight_only_quantize_amd import synth
from parity import assert_gemm_close, bf16_to_f64, bits_to_gpu, dev

pytestmark = pytest.mark.gpu


class Layer:
    """One projection: oracle-quantized NVFP4 weight + LoRA, host and GPU copies."""

    def __init__(self, n, k, r, seed, row_sigma=0.5, lora_scale=2.0):
        w = synth.weight_bf16(n, k, seed=seed, row_lognormal_sigma=row_sigma)
        self.packed, self.scales, self.s_t = oracle.nvfp4_quantize(synth.bf16_bits(w), threads=16)
        self.n, self.k, self.r, self.lam = n, k, r, lora_scale
        self.wq = q.NVFP4Weight(torch.from_numpy(self.packed).to(dev()),
                                torch.from_numpy(self.scales).to(dev()),
                                torch.tensor([self.s_t], dtype=torch.float32, device=dev()))
        if r:
            a, b = synth.lora_bf16(n, k, r, seed=seed + 7)
            self.a_bits, self.b_bits = synth.bf16_bits(a), synth.bf16_bits(b)
            self.a, self.b = a.to(dev()), b.to(dev())
        else:
            self.a_bits = self.b_bits = self.a = self.b = None

    def gpu(self, x_gpu):
        y = q.w4a16_lora_gemm(x_gpu, self.wq, self.a, self.b, self.lam)
        torch.cuda.synchronize()
        return y

    def ref(self, x_bits, rows=None):
        return oracle.w4a16_lora_gemm(x_bits, self.packed, self.scales, self.s_t, self.a_bits,
                                      self.b_bits, self.lam, rows=rows, threads=16)


def _x(m, k, seed, outliers=0.005):
    return synth.bf16_bits(synth.activation_bf16(m, k, seed=seed, outlier_col_frac=outliers))


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 16, 17, 24, 32, 33, 64, 100, 256])
@pytest.mark.parametrize("nkr", [(96, 256, 16), (77, 512, 32), (130, 1024, 8), (64, 48, 4),
                                 (33, 80, 0), (200, 2048, 64), (5, 128, 4), (300, 1040, 24),
                                 (1000, 3600, 32), (256, 1024, 128)])
def test_small_shapes(m, nkr):
    n, k, r = nkr
    L = Layer(n, k, r, seed=100 + n + k + r)
    x = _x(m, k, seed=m * 7 + k)
    y = bf16_to_f64(L.gpu(bits_to_gpu(x)))
    assert_gemm_close(y, L.ref(x), f"m={m} n={n} k={k} r={r}")


@pytest.mark.parametrize("m", [1, 4, 20, 64, 200])
def test_strided_activations_and_output(m):
    n, k, r = 96, 512, 16
    L = Layer(n, k, r, seed=300)
    x = _x(m, k, seed=301)
    xw = torch.zeros((m, k + 64), dtype=torch.bfloat16, device=dev())
    xw[:, :k] = bits_to_gpu(x)
    yw = torch.full((m, n + 32), 7.0, dtype=torch.bfloat16, device=dev())
    q.w4a16_lora_gemm(xw[:, :k], L.wq, L.a, L.b, L.lam, out=yw[:, :n])
    torch.cuda.synchronize()
    assert_gemm_close(bf16_to_f64(yw[:, :n]), L.ref(x), "strided")
    assert torch.all(yw[:, n:] == 7.0)


@pytest.mark.parametrize("m", [1, 20, 70])
def test_very_wide_x_rows(m):
    """x rows 2^22 + 64 elements apart: past the main loop's 32-bit buffer
    offsets, so the m > 16 paths take their plain loop for all of K."""
    n, k, r = 96, 256, 8
    L = Layer(n, k, r, seed=350)
    x = _x(m, k, seed=351)
    ldx = (1 << 22) + 64
    xw = torch.zeros((m, ldx), dtype=torch.bfloat16, device=dev())
    xw[:, :k] = bits_to_gpu(x)
    y = q.w4a16_lora_gemm(xw[:, :k], L.wq, L.a, L.b, L.lam)
    torch.cuda.synchronize()
    assert_gemm_close(bf16_to_f64(y), L.ref(x), f"wide rows m={m}")
    del xw


@pytest.mark.parametrize("m", [1, 3, 16, 80])
def test_zero_input_zero_lora(m):
    n, k, r = 64, 256, 8
    L = Layer(n, k, r, seed=400)
    zero = torch.zeros((m, k), dtype=torch.bfloat16, device=dev())
    assert torch.all(L.gpu(zero) == 0)
    x = _x(m, k, seed=401)
    base = q.w4a16_lora_gemm(bits_to_gpu(x), L.wq)
    zb = torch.zeros_like(L.b)
    with_zero_b = q.w4a16_lora_gemm(bits_to_gpu(x), L.wq, L.a, zb, 2.0)
    torch.cuda.synchronize()
    assert torch.equal(base, with_zero_b)
    assert_gemm_close(bf16_to_f64(base), oracle.w4a16_lora_gemm(x, L.packed, L.scales, L.s_t), "r=0")


def test_config1_single_layer():
    L = Layer(2048, 2048, 16, seed=1001, row_sigma=0.0, lora_scale=32 / 16)
    x = _x(1, 2048, seed=1002, outliers=0.0)
    assert_gemm_close(bf16_to_f64(L.gpu(bits_to_gpu(x))), L.ref(x), "config1")


@pytest.mark.parametrize("proj", synth.PROJ_ORDER)
def test_config2_7b_layer(proj):
    # every row and column at each decode batch
    n, k = synth.QWEN25_7B[proj]
    L = Layer(n, k, 32, seed=synth.seed_for(1002, proj))
    for m in (1, 8, 64):
        x = _x(m, k, seed=synth.seed_for(1002, proj, m))
        y = bf16_to_f64(L.gpu(bits_to_gpu(x)))
        assert_gemm_close(y, L.ref(x), f"{proj} m={m}")


@pytest.mark.parametrize("r", [8, 128])
def test_7b_lora_rank_sweep_ends(r):
    # the ends of the bench's LoRA-rank sweep at the 7B up projection
    n, k = synth.QWEN25_7B["up"]
    L = Layer(n, k, r, seed=synth.seed_for(1005, "up", r), lora_scale=64 / r)
    for m in (1, 8, 64):
        x = _x(m, k, seed=synth.seed_for(1005, "x", m))
        y = bf16_to_f64(L.gpu(bits_to_gpu(x)))
        rows = None if m <= 8 else [0, 17, 63]
        ref = L.ref(x, rows=rows)
        assert_gemm_close(y if rows is None else y[rows], ref, f"up r={r} m={m}")


@pytest.mark.parametrize("proj", synth.PROJ_ORDER)
def test_config3_32b_batched_decode(proj):
    # M 16 and 64 (decode kernels): every row; M 128 and 256 (MFMA tiles of
    # 128 rows): every 8th row, each at another offset inside its 16-row
    # MFMA tile, and the last -- all N columns, so every output tile is seen
    n, k = synth.QWEN25_32B[proj]
    L = Layer(n, k, 32, seed=synth.seed_for(1003, proj))
    for m in (16, 64, 128, 256):
        x = _x(m, k, seed=synth.seed_for(1003, proj, m))
        y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=dev())
        q.w4a16_lora_gemm(bits_to_gpu(x), L.wq, L.a, L.b, L.lam, out=y)
        torch.cuda.synchronize()
        y = bf16_to_f64(y)
        rows = None if m <= 64 else sorted(set([8 * i + (i % 8) for i in range(m // 8)] + [m - 1]))
        assert_gemm_close(y if rows is None else y[rows], L.ref(x, rows=rows), f"{proj} m={m}")


def tile_rows(m, tile=128):
    """One row from every `tile`-row block (at an offset that moves from block
    to block), plus the first and the last row."""
    rows = {0, m - 1}
    for t in range((m + tile - 1) // tile):
        rows.add(min(m - 1, t * tile + (37 * t + 11) % tile))
    return sorted(rows)


@pytest.fixture(scope="module")
def config4_gate_up():
    """The fused gate/up weight of the 32B layer: one NVFP4 tensor [2N, K]
    (one tensor scale), A = [A_gate; A_up] and the block-diagonal B."""
    n, k = synth.QWEN25_32B["gate"]
    r = 32
    w = synth.weight_bf16(2 * n, k, seed=synth.seed_for(1004, "gate_up"), row_lognormal_sigma=0.5)
    packed, scales, s_t = oracle.nvfp4_quantize(synth.bf16_bits(w), threads=16)
    del w
    ag, bg = synth.lora_bf16(n, k, r, seed=synth.seed_for(1004, "gate_lora"))
    au, bu = synth.lora_bf16(n, k, r, seed=synth.seed_for(1004, "up_lora"))
    a = torch.cat([ag, au], 0)
    b = torch.zeros((2 * n, 2 * r), dtype=torch.bfloat16)
    b[:n, :r] = bg
    b[n:, r:] = bu
    return packed, scales, s_t, a, b


def _prefill_check(m, k, packed, scales, s_t, a, b, lam, seed, what):
    n = packed.shape[0]
    wq = q.NVFP4Weight(torch.from_numpy(packed).to(dev()), torch.from_numpy(scales).to(dev()),
                       torch.tensor([s_t], dtype=torch.float32, device=dev()))
    x = _x(m, k, seed=seed)
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=dev())  # an unwritten tile stays NaN
    q.w4a16_lora_gemm(bits_to_gpu(x), wq, a.to(dev()), b.to(dev()), lam, out=y)
    torch.cuda.synchronize()
    rows = tile_rows(m)
    yr = bf16_to_f64(y[rows])
    del y, wq
    ref = oracle.w4a16_lora_gemm(x, packed, scales, s_t, synth.bf16_bits(a), synth.bf16_bits(b), lam,
                                 rows=rows, threads=16)
    assert_gemm_close(yr, ref, f"{what} m={m}")


@pytest.mark.parametrize("m", [2048, 8192])
def test_config4_prefill_fused_gate_up(m, config4_gate_up):
    packed, scales, s_t, a, b = config4_gate_up
    _prefill_check(m, packed.shape[1] * 2, packed, scales, s_t, a, b, 2.0, synth.seed_for(1004, "x", m), "gate_up")


@pytest.mark.parametrize("m", [2048, 8192])
@pytest.mark.parametrize("proj", ["q", "k", "v", "o", "down"])
def test_config4_prefill_projection(m, proj):
    # q/k/v/o [5120|1024, 5120] (k and v at M = 2048 split K) and down [5120, 27648]
    n, k = synth.QWEN25_32B[proj]
    w = synth.weight_bf16(n, k, seed=synth.seed_for(1004, proj), row_lognormal_sigma=0.5)
    packed, scales, s_t = oracle.nvfp4_quantize(synth.bf16_bits(w), threads=16)
    del w
    a, b = synth.lora_bf16(n, k, 32, seed=synth.seed_for(1004, proj, "lora"))
    _prefill_check(m, k, packed, scales, s_t, a, b, 2.0, synth.seed_for(1004, "x", proj, m), proj)


def test_gpu_quantizer_feeds_gemm():
    # end to end on the GPU: quantize with the HIP quantizer, multiply, compare
    n, k, r, m = 512, 3584, 32, 8
    w = synth.weight_bf16(n, k, seed=77, row_lognormal_sigma=0.5)
    wq = q.nvfp4_quantize(w.to(dev()))
    a, b = synth.lora_bf16(n, k, r, seed=78)
    x = _x(m, k, seed=79)
    y = q.w4a16_lora_gemm(bits_to_gpu(x), wq, a.to(dev()), b.to(dev()), 2.0)
    torch.cuda.synchronize()
    packed, scales, s_t = oracle.nvfp4_quantize(synth.bf16_bits(w))
    ref = oracle.w4a16_lora_gemm(x, packed, scales, s_t, synth.bf16_bits(a), synth.bf16_bits(b), 2.0)
    assert_gemm_close(bf16_to_f64(y), ref, "quantize->gemm")


def test_shared_workspace_sequence_is_deterministic():
    """One workspace, filled with garbage first, serves a mixed sequence of
    calls (decode with and without split K and LoRA, and the large-m path with
    split K, the splits meeting in the launch with and without LoRA -- the
    split tiles' counters start from garbage -- or in a reduce launch); each
    output equals the one from a fresh workspace bit for bit."""
    cases = [(1, 3584, 3584, 32), (8, 512, 3584, 32), (64, 18944 // 4, 3584, 32), (33, 1000, 3600, 24),
             (1, 3584, 18944 // 2, 0), (100, 512, 1024, 16), (16, 77, 512, 8), (64, 3584, 3584, 32),
             (200, 520, 2048, 0), (1000, 2000, 1024, 0)]
    layers, xs = [], []
    for i, (m, n, k, r) in enumerate(cases):
        layers.append(Layer(n, k, r, seed=900 + i))
        xs.append(bits_to_gpu(_x(m, k, seed=950 + i)))
    need = max(q.w4a16_lora_gemm_workspace_size(m, n, k, r) for m, n, k, r in cases)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=dev())
    fresh = [q.w4a16_lora_gemm(x, L.wq, L.a, L.b, L.lam) for x, L in zip(xs, layers)]
    for _ in range(3):
        for i, (x, L) in enumerate(zip(xs, layers)):
            y = q.w4a16_lora_gemm(x, L.wq, L.a, L.b, L.lam, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(y, fresh[i]), f"case {cases[i]}"
    for i in (0, 3):
        m, n, k, r = cases[i]
        assert_gemm_close(bf16_to_f64(fresh[i]), layers[i].ref(synth.bf16_bits(xs[i].cpu())), f"case {cases[i]}")


@pytest.mark.parametrize("m,n,k,r", [
    (300, 1000, 1280, 16),  # 10 blocks, two splits: 5 per split rounds to 6 (6 + 4)
    (200, 520, 3328, 32),   # 26 blocks in splits of 6, 6, 6, 6, 2 (partial chunks)
    (300, 300, 768, 8),     # one split of 6 blocks (a chunk and a half), ragged n and m
    (129, 264, 384, 4),     # K % 256 == 128: scales by plain loads; 8 rows in the last n tile
    (70, 1000, 2048, 24),   # 16 blocks in 4 splits of 4; 232 rows in the last n tile
    (300, 1000, 2048, 0),   # split K without LoRA, the splits summed by a reduce launch
    (1000, 2000, 1024, 0),  # two splits meeting in the launch without LoRA (counters cleared by a launch of their own)
])
def test_prefill_scale_chunks(m, n, k, r):
    """The prefill K loop takes the scales by LDS DMA, four blocks at a time,
    when K is a multiple of 256 and the split starts at an even block: partial
    chunks at the end of a split, split sizes rounded up to even, weight tiles
    with rows past n, and the plain-load path for the other K.  The splits of
    a tile meet in the launch (the last to arrive sums them: the two-split
    cases) or in a reduce launch (the tiles with more splits), with and
    without LoRA."""
    L = Layer(n, k, r, seed=1300 + m + n + k)
    x = _x(m, k, seed=1301 + m + k)
    y = bf16_to_f64(L.gpu(bits_to_gpu(x)))
    assert_gemm_close(y, L.ref(x), f"m={m} n={n} k={k} r={r}")


@pytest.mark.parametrize("s_t", [1e-39, 1e-30, 1e-18])
@pytest.mark.parametrize("m", [257, 300, 1000])
def test_tiny_tensor_scale(m, s_t):
    """The prefill path folds lambda / s_t into its accumulation only while
    that factor is finite and moderate; for a subnormal or tiny s_t the LoRA
    term is added in the epilogue (split and unsplit K both: 300 x 1000 x 2048
    splits, 257 x 96 x 256 does not; at m = 1000 the four splits of 1000 x 1000 x
    2048 meet in the launch, at m = 300 in a reduce launch).  Decode (m <= 256)
    applies s_t apart."""
    for n, k, r in ((96, 256, 16), (1000, 2048, 32)):
        L = Layer(n, k, r, seed=900 + n + m)
        L.s_t = np.float32(s_t)
        L.wq = q.NVFP4Weight(L.wq.packed, L.wq.scales, torch.tensor([L.s_t], dtype=torch.float32, device=dev()))
        x = _x(m, k, seed=m + 3 * k)
        y = bf16_to_f64(L.gpu(bits_to_gpu(x)))
        assert_gemm_close(y, L.ref(x), f"m={m} n={n} k={k} r={r} s_t={s_t}")
    # decode path, same scales
    L = Layer(96, 256, 16, seed=990)
    L.s_t = np.float32(s_t)
    L.wq = q.NVFP4Weight(L.wq.packed, L.wq.scales, torch.tensor([L.s_t], dtype=torch.float32, device=dev()))
    x = _x(8, 256, seed=991)
    assert_gemm_close(bf16_to_f64(L.gpu(bits_to_gpu(x))), L.ref(x), f"decode s_t={s_t}")
