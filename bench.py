#!/usr/bin/env python3
"""Benchmark of the QeRL rollout-phase linear layer on one MI355X.

One *step* is the decode pass of two synthetic decoder layers through every
operation of the hot path:

  * a Qwen2.5-7B-shaped layer at decode batch M in {1, 8, 64}, and
  * a Qwen2.5-32B-shaped layer at batched-rollout M in {16, 64},

each as  AQN RMSNorm -> q|k|v,  o,  AQN RMSNorm -> gate|up,  down  (NVFP4
W4A16 + LoRA r=32, alpha=64 on all seven projections; o and down take
synthetic inputs, where attention and the MLP activation would sit).

The AQN noise is that of one RL step (sigma of stage 3 of the exponential
schedule 1e-2 -> 5e-4 over 10 stages): drawn once, as every decode step of a
rollout uses the same noisy norm weight; each norm runs inside the call of the
projections that read it (qerl_rmsnorm_w4a16_lora_gemm_multi).  Weights are
cold: rotating copies of each layer's NVFP4 weights and LoRA (about 1.1 GB per
layer, far above the 256 MB Infinity Cache) so that no weight is re-read from
cache.  The steps run as one captured HIP graph.

``value`` = algorithmic bytes of a step / wall time of a step (GB/s), inputs
resident in HBM.  Algorithmic bytes per projection call:
    N*K/2 + N*K/16 + 4 (NVFP4 weight) + 2*r*(K + N) (LoRA) + 2*M*(K + N) (x, y)
and per norm: 2*M*H (x) + 4*H (weight) + 2*M*H (BF16 out).

Other legs in the same JSON line: ``roofline`` (the decode GEMM call class
with the larger share of the step), ``decode_32b_large_m`` (the 32B layer at
M 128 and 256, past the ridge: both roofline fractions), ``prefill`` (32B
layer, M in {2048, 8192}, TFLOP/s), ``quantizer`` (one 32B layer; the whole
64-layer 32B model streamed layer by layer; the 2048 x 2048 single layer),
``single_layer_2048`` (the W4A16 + LoRA GEMM of that layer at M = 1),
``aqn_rmsnorm`` (the norm alone), ``cpu_baseline`` (the CPU oracle on a
bounded sample of the decode workload) and the comparison and update-phase
legs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import nvfp4_weight_only_quantize_amd as q  # noqa: E402
from nvfp4_weight_only_quantize_amd import synth  # noqa: E402

METRIC = "W4A16-NVFP4+LoRA GEMM: decode HBM GB/s (%peak), prefill TFLOPS (%MFMA peak)"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
PREFILL_MS = (2048, 8192)
RANK, ALPHA = 32, 64
SIGMA0, SIGMA1, STAGES, EPS = 1e-2, 5e-4, 10, 1e-6
RL_STEP = 3  # the RL step (noise stage) the decode steps belong to
SEED = 1002

# the decoder layers of a step: shapes, hidden and intermediate widths,
# decode batches, master seed, cold copies
LAYER_7B = dict(name="qwen2.5-7b", shapes=synth.QWEN25_7B, hidden=3584, inter=18944, ms=(1, 8, 64), seed=1002,
                copies=8)
LAYER_32B = dict(name="qwen2.5-32b", shapes=synth.QWEN25_32B, hidden=5120, inter=27648, ms=(16, 64), seed=1003,
                 copies=4)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_bytes(m, n, k, r):
    return n * k // 2 + n * k // 16 + 4 + 2 * r * (k + n) + 2 * m * (k + n)


def gemm_flops(m, n, k, r):
    return 2 * m * n * k + 2 * m * r * (k + n)


def norm_bytes(m, h):
    return 2 * m * h + 4 * h + 2 * m * h


def pct(v, lo, hi):
    """(p10, p50, p90) of a list."""
    a = np.sort(np.asarray(v, dtype=np.float64))
    return tuple(float(np.percentile(a, x)) for x in (lo, 50, hi))


class Proj:
    """One NVFP4 projection with its LoRA (GPU)."""

    def __init__(self, wq, a, b):
        self.wq, self.a, self.b = wq, a, b

    def clone(self):
        return Proj(q.NVFP4Weight(self.wq.packed.clone(), self.wq.scales.clone(),
                                  self.wq.tensor_scale.clone()), self.a.clone(), self.b.clone())


def make_layer(shapes, seed, dev, r=RANK, row_sigma=0.5, outlier_rows=0.0):
    """Quantize a synthetic BF16 layer on the GPU; returns {name: Proj}."""
    layer = {}
    for name in synth.PROJ_ORDER:
        n, k = shapes[name]
        w = synth.weight_bf16(n, k, seed=synth.seed_for(seed, name), row_lognormal_sigma=row_sigma,
                              outlier_row_frac=outlier_rows, device=dev)
        wq = q.nvfp4_quantize(w)
        del w
        a, b = synth.lora_bf16(n, k, r, seed=synth.seed_for(seed, name, "lora"), device=dev)
        layer[name] = Proj(wq, a, b)
    return layer


class DecodeLayer:
    """Buffers and the launch sequence of one decoder layer's decode pass."""

    def __init__(self, cfg, dev, copies=None, launch="fused"):
        self.cfg, self.dev, self.launch = cfg, dev, launch
        self.shapes, self.ms = cfg["shapes"], cfg["ms"]
        h, inter, seed = cfg["hidden"], cfg["inter"], cfg["seed"]
        self.h = h
        base = make_layer(self.shapes, seed, dev)
        ncopy = copies or cfg["copies"]
        self.copies = [base] + [{k: p.clone() for k, p in base.items()} for _ in range(ncopy - 1)]
        mmax = max(self.ms)
        self.h_attn = synth.activation_bf16(mmax, h, synth.seed_for(seed, "h_attn"), 0.005, device=dev)
        self.h_mlp = synth.activation_bf16(mmax, h, synth.seed_for(seed, "h_mlp"), 0.005, device=dev)
        self.x_o = synth.activation_bf16(mmax, h, synth.seed_for(seed, "x_o"), 0.005, device=dev)
        self.x_down = synth.activation_bf16(mmax, inter, synth.seed_for(seed, "x_down"), 0.005, device=dev)
        self.w_attn = synth.norm_weight_f32(h, synth.seed_for(seed, "w_attn"), device=dev)
        self.w_mlp = synth.norm_weight_f32(h, synth.seed_for(seed, "w_mlp"), device=dev)
        self.x_attn = torch.empty((mmax, h), dtype=torch.bfloat16, device=dev)
        self.x_mlp = torch.empty((mmax, h), dtype=torch.bfloat16, device=dev)
        self.y = {name: torch.empty((mmax, n), dtype=torch.bfloat16, device=dev)
                  for name, (n, _k) in self.shapes.items()}
        ws = max(q.w4a16_lora_gemm_workspace_size(m, n, k, RANK) for n, k in self.shapes.values() for m in self.ms)
        for group in (("q", "k", "v"), ("gate", "up")):
            for m in self.ms:
                shp = [(self.shapes[g][0], RANK) for g in group]
                ws = max(ws, q.w4a16_lora_gemm_multi_workspace_size(m, self.shapes[group[0]][1], shp),
                         q.rmsnorm_w4a16_lora_gemm_multi_workspace_size(m, self.shapes[group[0]][1], shp))
        # one workspace per concurrent GEMM (calls that overlap must not share one)
        self.ws = [torch.empty(max(ws, 256), dtype=torch.uint8, device=dev) for _ in range(3)]
        # side streams for the independent projections (default priority)
        self.side = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
        # AQN: the noise of one RL step is drawn once and every decode step of
        # the rollout reuses it (the fused launches take the noisy weight; the
        # standalone norm redraws the same vector on each call)
        self.sigma = q.aqn_sigma(RL_STEP, STAGES, SIGMA0, SIGMA1)
        self.wn_attn = q.aqn_noisy_weight(self.w_attn, self.sigma, seed, RL_STEP, 0)
        self.wn_mlp = q.aqn_noisy_weight(self.w_mlp, self.sigma, seed, RL_STEP, 1)
        self.norm("attn", mmax)
        self.norm("mlp", mmax)

    def inputs_of(self, name):
        return {"q": self.x_attn, "k": self.x_attn, "v": self.x_attn, "o": self.x_o,
                "gate": self.x_mlp, "up": self.x_mlp, "down": self.x_down}[name]

    def gemm(self, name, m, c, slot=0):
        p = self.copies[c][name]
        q.w4a16_lora_gemm(self.inputs_of(name)[:m], p.wq, p.a, p.b, ALPHA / RANK,
                          out=self.y[name][:m], workspace=self.ws[slot])

    def norm_gemm_multi(self, which, names, m, c):
        """The AQN RMSNorm `which` and the projections `names` that read its
        output, in one call."""
        src, wn = (self.h_attn, self.wn_attn) if which == "attn" else (self.h_mlp, self.wn_mlp)
        segs = [(self.copies[c][n].wq, self.copies[c][n].a, self.copies[c][n].b, ALPHA / RANK) for n in names]
        q.rmsnorm_w4a16_lora_gemm_multi(src[:m], wn, EPS, segs, outs=[self.y[n][:m] for n in names],
                                        workspace=self.ws[0])

    def norm(self, which, m):
        src, w, dst, layer = ((self.h_attn, self.w_attn, self.x_attn, 0) if which == "attn"
                              else (self.h_mlp, self.w_mlp, self.x_mlp, 1))
        q.aqn_rmsnorm(src[:m], w, EPS, self.sigma, self.cfg["seed"], RL_STEP, layer, want_f32=False,
                      y_bf16=dst[:m])

    def step_m(self, s, m, mi, on_gemm=None):
        """The layer's decode pass at batch m (copy chosen by step s)."""
        c = (len(self.ms) * s + mi) % len(self.copies)
        fused = on_gemm is None and self.launch == "fused"
        if not fused:
            self.norm("attn", m)
        if on_gemm is None and self.launch != "serial":
            # q, k and v read the same normed input and nothing else: one call
            # with the norm (or side by side on side streams after it); o
            # waits for all three (in a real layer attention sits in between),
            # as the MLP waits for o
            if fused:
                self.norm_gemm_multi("attn", ("q", "k", "v"), m, c)
            else:
                self._parallel(("q", "k", "v"), m, c)
            self.gemm("o", m, c)
        else:
            for name in ("q", "k", "v", "o"):
                self._g(name, m, c, on_gemm)
        if not fused:
            self.norm("mlp", m)
        if on_gemm is None and self.launch != "serial":
            if fused:
                self.norm_gemm_multi("mlp", ("gate", "up"), m, c)
            else:
                self._parallel(("gate", "up"), m, c)  # down waits for both
            self.gemm("down", m, c)
        else:
            for name in ("gate", "up", "down"):
                self._g(name, m, c, on_gemm)

    def step(self, s, on_gemm=None):
        for mi, m in enumerate(self.ms):
            self.step_m(s, m, mi, on_gemm)

    def _parallel(self, names, m, c):
        """names[0] on the current stream, the rest on side streams, joined
        back into the current stream; each call has its own workspace."""
        main = torch.cuda.current_stream()
        for i, name in enumerate(names[1:]):
            st = self.side[i]
            st.wait_stream(main)
            with torch.cuda.stream(st):
                self.gemm(name, m, c, slot=i + 1)
        self.gemm(names[0], m, c, slot=0)
        for st in self.side[:len(names) - 1]:
            main.wait_stream(st)

    def _g(self, name, m, c, on_gemm):
        if on_gemm is None:
            self.gemm(name, m, c)
        else:
            on_gemm(name, m, lambda: self.gemm(name, m, c))

    def bytes_m(self, m):
        return 2 * norm_bytes(m, self.h) + sum(gemm_bytes(m, n, k, RANK) for n, k in self.shapes.values())

    def step_bytes(self):
        return sum(self.bytes_m(m) for m in self.ms)


def warm_up(run, min_s=0.3):
    """Keep the GPU busy with run() for about min_s seconds before a leg's
    timed region, so it does not start on clocks still rising from idle (the
    first leg of a process measured up to 10% low otherwise): one timed run,
    then enough runs enqueued back to back, one synchronization at the end
    (a synchronization after every short run leaves the GPU mostly idle)."""
    t0 = time.perf_counter()
    run()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 1e-5)
    for _ in range(min(int(min_s / one), 20000)):
        run()
    torch.cuda.synchronize()


def time_graph(fn_steps, steps, warmup):
    """Capture `steps` calls of fn (and `warmup` separately) as HIP graphs;
    returns ms per step and the graphs."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn_steps(0, 1)  # eager pass: one-time setup (function attributes) before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g_warm, g_main = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_warm):
        fn_steps(0, max(warmup, 1))
    with torch.cuda.graph(g_main):
        fn_steps(warmup, steps)
    g_warm.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    g_main.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, (g_warm, g_main)


def replay_percentiles(fn, reps=120, warm=20):
    """fn() captured as one graph and replayed reps times, an event pair
    around each replay: (p10, p50, p90) in microseconds."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        g.replay()
        e1.record()
    torch.cuda.synchronize()
    del g
    return pct([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs], 10, 90)


def check_decode_parity(layers):
    """GPU outputs vs the CPU oracle: for each layer at its smallest M, the
    five projections behind a norm through the fused norm call (oracle:
    RMSNorm then the layer), and o and down as single calls.  Worst relative
    L2 error."""
    import oracle
    worst = 0.0
    for layer in layers:
        m = min(layer.ms)
        for which, names in (("attn", ("q", "k", "v")), ("mlp", ("gate", "up"))):
            layer.norm_gemm_multi(which, names, m, 0)
            torch.cuda.synchronize()
            src, wn = (layer.h_attn, layer.wn_attn) if which == "attn" else (layer.h_mlp, layer.wn_mlp)
            x = synth.bf16_bits(src[:m])
            for name in names:
                p = layer.copies[0][name]
                y = layer.y[name][:m].float().cpu().numpy().astype(np.float64)
                ref = oracle.rmsnorm_w4a16_lora_gemm(x, wn.cpu().numpy(), EPS, p.wq.packed.cpu().numpy(),
                                                     p.wq.scales.cpu().numpy(), np.float32(p.wq.tensor_scale.item()),
                                                     synth.bf16_bits(p.a), synth.bf16_bits(p.b), ALPHA / RANK,
                                                     threads=16)
                worst = max(worst, float(np.linalg.norm(y - ref) / np.linalg.norm(ref)))
        for name in ("o", "down"):
            p = layer.copies[0][name]
            x = synth.bf16_bits(layer.inputs_of(name)[:m])
            layer.gemm(name, m, 0)
            torch.cuda.synchronize()
            y = layer.y[name][:m].float().cpu().numpy().astype(np.float64)
            ref = oracle.w4a16_lora_gemm(x, p.wq.packed.cpu().numpy(), p.wq.scales.cpu().numpy(),
                                         np.float32(p.wq.tensor_scale.item()), synth.bf16_bits(p.a),
                                         synth.bf16_bits(p.b), ALPHA / RANK, threads=16)
            worst = max(worst, float(np.linalg.norm(y - ref) / np.linalg.norm(ref)))
    return worst


def host_cpu():
    """(threads the oracle may use here, CPU model name)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    # a GPU machine's share of the host is 16 threads, whatever the affinity mask shows
    return min(16, avail), model


def cpu_baseline(layers, budget_s: float):
    """The CPU oracle on the decode step's projections: the 7B layer's seven
    at M = 1, 8, 64, then the 32B layer's at M = 16, 64 (one whole step of
    GEMM work), stopping early once the time budget is spent.  Same
    algorithmic-bytes accounting as the GPU."""
    import oracle
    threads, model = host_cpu()
    done_bytes, t_used, sample = 0, 0.0, []
    for L in layers:
        host = {}
        for name in synth.PROJ_ORDER:
            p = L.copies[0][name]
            host[name] = (p.wq.packed.cpu().numpy(), p.wq.scales.cpu().numpy(),
                          np.float32(p.wq.tensor_scale.item()), synth.bf16_bits(p.a), synth.bf16_bits(p.b))
        xs = {name: synth.bf16_bits(L.inputs_of(name)[:max(L.ms)]) for name in synth.PROJ_ORDER}
        for m in L.ms:
            for name in synth.PROJ_ORDER:
                if t_used > budget_s:
                    break
                n, k = L.shapes[name]
                packed, scales, st, a, b = host[name]
                t0 = time.perf_counter()
                oracle.w4a16_lora_gemm(xs[name][:m], packed, scales, st, a, b, ALPHA / RANK, threads=threads)
                t_used += time.perf_counter() - t0
                done_bytes += gemm_bytes(m, n, k, RANK)
                sample.append(f"{L.cfg['name']} {name}@M={m}")
        del host, xs
    return {"value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": model,
            "sample": f"fp64 oracle W4A16+LoRA, {len(sample)} projection calls of the step ({sample[0]} .. "
                      f"{sample[-1]}; {done_bytes / 1e6:.1f} MB algorithmic, {t_used:.1f} s)"}


def _graph_us(fn, reps):
    """Average microseconds of fn(s) for s < reps, captured as one HIP graph
    (after one eager pass) and replayed once between two events."""
    fn(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(reps):
            fn(s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / reps


def bf16_lora_leg(layer: DecodeLayer, reps: int = 5):
    """The seven 7B projections at each decode M, one after another on one
    stream, cold weights rotating: this library's W4A16 + LoRA against torch's
    BF16 GEMM + the same LoRA (hipBLASLt; BF16 weights of the same shapes, one
    copy per cold copy of the NVFP4 weights).  The pages' comparison is NVFP4
    rollout against 16-bit LoRA rollout."""
    dev = layer.dev
    ncopy = len(layer.copies)
    dense = []
    for c in range(ncopy):
        dense.append({name: (torch.randn(n, k, device=dev, dtype=torch.bfloat16) * 0.02)
                      for name, (n, k) in layer.shapes.items()})
    lam = ALPHA / RANK
    out = {}
    for m in layer.ms:
        def ours(s, m=m):
            c = (s * 3 + 1) % ncopy
            for name in synth.PROJ_ORDER:
                layer.gemm(name, m, c)

        def torch_bf16(s, m=m):
            c = (s * 3 + 1) % ncopy
            for name in synth.PROJ_ORDER:
                p, x = layer.copies[c][name], layer.inputs_of(name)[:m]
                y = torch.nn.functional.linear(x, dense[c][name])
                y.add_(torch.nn.functional.linear(torch.nn.functional.linear(x, p.a), p.b), alpha=lam)

        t_ours, t_bf16 = _graph_us(ours, reps), _graph_us(torch_bf16, reps)
        out[f"M={m}"] = {"w4a16_lora_us": round(t_ours, 2), "bf16_lora_us": round(t_bf16, 2),
                         "speedup": round(t_bf16 / t_ours, 3)}
    del dense
    torch.cuda.empty_cache()
    return out


def lora_rank_leg(layer: DecodeLayer, ranks=(8, 16, 32, 64, 128), reps: int = 5):
    """The seven 7B projections at each decode M with LoRA ranks 8..128 (cold
    NVFP4 weights rotating as in the step; one LoRA per rank and copy)."""
    dev = layer.dev
    ncopy = len(layer.copies)
    out = {}
    for r in ranks:
        loras = [{name: synth.lora_bf16(n, k, r, seed=synth.seed_for(SEED, name, "rank", r, c), device=dev)
                  for name, (n, k) in layer.shapes.items()} for c in range(ncopy)]
        ws = torch.empty(max(q.w4a16_lora_gemm_workspace_size(max(layer.ms), n, k, r)
                             for n, k in layer.shapes.values()), dtype=torch.uint8, device=dev)
        row = {}
        for m in layer.ms:
            def fn(s, m=m):
                c = (s * 3 + 2) % ncopy
                for name in synth.PROJ_ORDER:
                    p = layer.copies[c][name]
                    a, b = loras[c][name]
                    q.w4a16_lora_gemm(layer.inputs_of(name)[:m], p.wq, a, b, ALPHA / r,
                                      out=layer.y[name][:m], workspace=ws)

            t = _graph_us(fn, reps)
            b_m = sum(gemm_bytes(m, *layer.shapes[name], r) for name in synth.PROJ_ORDER)
            row[f"M={m}"] = {"us": round(t, 2), "GB/s": round(b_m / (t * 1e-6) / 1e9, 1)}
        out[f"r={r}"] = row
        del loras, ws
    torch.cuda.empty_cache()
    return out


def prefill_leg(dev, reps):
    shapes = dict(synth.QWEN25_32B)
    layer = make_layer(shapes, 1004, dev)
    # fused gate/up: one NVFP4 tensor [2N, K] (its own tensor scale) with a
    # block-diagonal rank-64 LoRA
    n, k = shapes["gate"]
    w = synth.weight_bf16(2 * n, k, seed=synth.seed_for(1004, "gate_up"), row_lognormal_sigma=0.5, device=dev)
    gu = q.nvfp4_quantize(w)
    del w
    a = torch.cat([layer["gate"].a, layer["up"].a], 0)
    b = torch.zeros((2 * n, 2 * RANK), dtype=torch.bfloat16, device=dev)
    b[:n, :RANK] = layer["gate"].b
    b[n:, RANK:] = layer["up"].b
    projs = {"q": (layer["q"], RANK), "k": (layer["k"], RANK), "v": (layer["v"], RANK),
             "o": (layer["o"], RANK), "gate_up": (Proj(gu, a, b), 2 * RANK), "down": (layer["down"], RANK)}
    out, tot_flops, tot_t = {}, 0, 0.0
    for m in PREFILL_MS:
        xk = {kk: synth.activation_bf16(m, kk, synth.seed_for(1004, "x", m, kk), 0.005, device=dev)
              for kk in {5120, 27648}}
        ys = {nm: torch.empty((m, p.wq.shape[0]), dtype=torch.bfloat16, device=dev) for nm, (p, _r) in projs.items()}
        ws = torch.empty(max(q.w4a16_lora_gemm_workspace_size(m, p.wq.shape[0], p.wq.shape[1], r)
                             for p, r in projs.values()), dtype=torch.uint8, device=dev)

        def run():
            for nm, (p, r) in projs.items():
                q.w4a16_lora_gemm(xk[p.wq.shape[1]], p.wq, p.a, p.b, ALPHA / RANK, out=ys[nm], workspace=ws)

        warm_up(run)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        flops = sum(gemm_flops(m, p.wq.shape[0], p.wq.shape[1], r) for p, r in projs.values())
        out[f"M={m}"] = {"ms": t * 1e3, "tflops": flops / t / 1e12,
                         "frac": flops / t / 1e12 / BF16_MFMA_PEAK_TFLOPS}
        tot_flops += flops
        tot_t += t
        del xk, ys, ws
    # the layer aggregate over both M: sum of flops / sum of time
    out.update({"value": tot_flops / tot_t / 1e12, "unit": "TFLOP/s",
                "frac": tot_flops / tot_t / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                "workload": "Qwen2.5-32B-shaped layer, q/k/v/o, fused gate|up [55296, 5120] (rank-64 "
                            "block-diagonal LoRA) and down, NVFP4 W4A16 + LoRA, M in {2048, 8192}"})
    return out


def quantizer_leg(dev, reps):
    shapes = synth.QWEN25_32B
    ws = torch.empty(q.nvfp4_quantize_workspace_size(1, 16), dtype=torch.uint8, device=dev)
    ws_in, outs, elems = {}, {}, 0
    for name in synth.PROJ_ORDER:
        n, k = shapes[name]
        ws_in[name] = synth.weight_bf16(n, k, seed=synth.seed_for(1005, name), outlier_row_frac=0.001, device=dev)
        outs[name] = q.NVFP4Weight(torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
                                   torch.empty((n, k // 16), dtype=torch.uint8, device=dev),
                                   torch.empty(1, dtype=torch.float32, device=dev))
        elems += n * k

    def run():
        for name in synth.PROJ_ORDER:
            q.nvfp4_quantize(ws_in[name], out=outs[name], workspace=ws, check_finite=False)

    def timed(fn):
        warm_up(fn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t = timed(run)
    gbs = elems * 4.5625 / t / 1e9
    # one pass: the tensor scale supplied (each tensor's own, from the run
    # above), so only the encode pass runs: 2.5625 B per element
    scales_in = {name: outs[name].tensor_scale.clone() for name in synth.PROJ_ORDER}

    def run_one_pass():
        for name in synth.PROJ_ORDER:
            q.nvfp4_quantize(ws_in[name], tensor_scale_in=scales_in[name], out=outs[name], check_finite=False)

    t1 = timed(run_one_pass)
    gbs1 = elems * 2.5625 / t1 / 1e9
    return {"workload": f"BF16->NVFP4 of one Qwen2.5-32B-shaped layer (7 tensors, {elems / 1e9:.3f} G elements)",
            "ms": t * 1e3, "GB/s": gbs, "frac": gbs / HBM_PEAK_GBS,
            "one_pass_tensor_scale_in": {"ms": t1 * 1e3, "GB/s": gbs1, "frac": gbs1 / HBM_PEAK_GBS,
                                         "bytes_per_element": 2.5625}}


def model_quantizer_leg(dev, layers=64, verify_layers=(0, 37), verify=True):
    """The whole 64-layer Qwen2.5-32B-shaped weight set quantized layer by
    layer: each layer's seven BF16 tensors are generated on the GPU (W ~ N(0,
    0.02^2), 0.1% outlier rows x20), quantized into the resident NVFP4 model,
    and freed.  GPU time = the quantize calls of every layer, event-timed per
    layer; the whole pass (generation included) is timed too.  A seeded
    sample of layers is compared bit for bit with the CPU oracle.  Memory: the
    quantized model (plus the BF16 embedding and lm_head of 152064 x 5120,
    kept in 16 bits) against the all-BF16 model."""
    shapes = synth.QWEN25_32B
    ws = torch.empty(q.nvfp4_quantize_workspace_size(1, 16), dtype=torch.uint8, device=dev)
    model, evs, checks = [], [], []
    elems = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for li in range(layers):
        ws_in = {}
        for name in synth.PROJ_ORDER:
            n, k = shapes[name]
            ws_in[name] = synth.weight_bf16(n, k, seed=synth.seed_for(1005, li, name), outlier_row_frac=0.001,
                                            device=dev)
        outs = {name: q.NVFP4Weight(torch.empty((w.shape[0], w.shape[1] // 2), dtype=torch.uint8, device=dev),
                                    torch.empty((w.shape[0], w.shape[1] // 16), dtype=torch.uint8, device=dev),
                                    torch.empty(1, dtype=torch.float32, device=dev)) for name, w in ws_in.items()}
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for name in synth.PROJ_ORDER:
            q.nvfp4_quantize(ws_in[name], out=outs[name], workspace=ws, check_finite=False)
        e1.record()
        evs.append((e0, e1))
        elems += sum(w.numel() for w in ws_in.values())
        if verify and li in verify_layers:
            checks.append((li, {name: synth.bf16_bits(w) for name, w in ws_in.items()}))
        model.append(outs)
        del ws_in
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_q = sum(e0.elapsed_time(e1) for e0, e1 in evs) * 1e-3
    bad = []
    if verify:
        import oracle
        threads, _ = host_cpu()
        for li, bits in checks:
            for name in synth.PROJ_ORDER:
                op, osc, ot = oracle.nvfp4_quantize(bits[name], threads=threads)
                g = model[li][name]
                if not (np.array_equal(g.packed.cpu().numpy(), op) and np.array_equal(g.scales.cpu().numpy(), osc)
                        and np.float32(g.tensor_scale.item()) == ot):
                    bad.append(f"layer {li} {name}")
    emb = 2 * 152064 * 5120  # embedding and lm_head elements, kept BF16
    q_bytes = sum(w.nbytes for L in model for w in L.values())
    ratio = (q_bytes + 2 * emb) / (2 * elems + 2 * emb)
    del model
    torch.cuda.empty_cache()
    gbs = elems * 4.5625 / t_q / 1e9
    return {"workload": f"whole Qwen2.5-32B-shaped model: {layers} layers x 7 tensors, {elems / 1e9:.2f} G elements "
                        "(62.4 GB BF16), generated, quantized and freed layer by layer",
            "quantize_ms": t_q * 1e3, "GB/s": gbs, "frac": gbs / HBM_PEAK_GBS,
            "wall_s_with_generation": wall, "nvfp4_bytes": q_bytes,
            "memory_ratio_vs_bf16": ratio, "memory_ratio_note": "NVFP4 layers + BF16 embedding and lm_head over "
                                                               "the all-BF16 model",
            "verified_layers": [li for li, _ in checks], "verify_mismatches": bad}


def single_layer_leg(dev, copies=128, reps=20):
    """The smallest instance: W [2048, 2048] (N(0, 0.02^2)), LoRA r = 16,
    alpha = 32, x [1, 2048].  The quantizer (GB/s at 4.5625 B/element) and
    the W4A16 + LoRA GEMM at M = 1 (GB/s of its algorithmic bytes), each over
    `copies` rotating cold copies in one graph."""
    n = k = 2048
    r = 16
    ws_q = torch.empty(q.nvfp4_quantize_workspace_size(n, k), dtype=torch.uint8, device=dev)
    ws_in = [synth.weight_bf16(n, k, seed=synth.seed_for(1001, "w", c), device=dev) for c in range(copies)]
    outs = [q.NVFP4Weight(torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
                          torch.empty((n, k // 16), dtype=torch.uint8, device=dev),
                          torch.empty(1, dtype=torch.float32, device=dev)) for _ in range(copies)]

    def quant():
        for c in range(copies):
            q.nvfp4_quantize(ws_in[c], out=outs[c], workspace=ws_q, check_finite=False)

    tq = _graph_ms(quant, 3) * 1e-3 / copies
    del ws_in
    a, b = synth.lora_bf16(n, k, r, seed=synth.seed_for(1001, "lora"), device=dev)
    loras = [(a.clone(), b.clone()) for _ in range(copies)]
    x = synth.activation_bf16(1, k, synth.seed_for(1001, "x"), device=dev)
    y = torch.empty((1, n), dtype=torch.bfloat16, device=dev)
    ws_g = torch.empty(q.w4a16_lora_gemm_workspace_size(1, n, k, r), dtype=torch.uint8, device=dev)

    def gemm():
        for c in range(copies):
            q.w4a16_lora_gemm(x, outs[c], loras[c][0], loras[c][1], 32 / r, out=y, workspace=ws_g)

    tg = _graph_ms(gemm, reps) * 1e-3 / copies
    p10, p50, p90 = replay_percentiles(lambda: q.w4a16_lora_gemm(x, outs[0], loras[0][0], loras[0][1], 32 / r,
                                                                 out=y, workspace=ws_g))
    gb = gemm_bytes(1, n, k, r)
    del outs, loras
    return {"workload": "W [2048, 2048] NVFP4, LoRA r = 16 (alpha 32), x [1, 2048]",
            "quantizer_us": tq * 1e6, "quantizer_GB/s": n * k * 4.5625 / tq / 1e9,
            "gemm_us": tg * 1e6, "gemm_GB/s": gb / tg / 1e9, "gemm_frac": gb / tg / 1e9 / HBM_PEAK_GBS,
            "gemm_single_call_us_p10_p50_p90": [p10, p50, p90],
            "note": "cold: rotating copies; a 2.5 MB call is bound by launch and ramp, not bandwidth"}


def aqn_leg(dev):
    """AQN RMSNorm on its own (qerl_aqn_rmsnorm: noise drawn, scale vector
    w + sigma z, BF16 output): bytes 2 M H (x) + 4 H (weight) + 2 M H (y)."""
    out = {}
    sigma = q.aqn_sigma(RL_STEP, STAGES, SIGMA0, SIGMA1)
    for m, h in ((1, 3584), (8192, 5120)):
        x = synth.activation_bf16(m, h, synth.seed_for(1006, "x", m), 0.005, device=dev)
        w = synth.norm_weight_f32(h, synth.seed_for(1006, "w", h), device=dev)
        y = torch.empty((m, h), dtype=torch.bfloat16, device=dev)
        calls = 20  # per graph, so the per-call time is not one graph launch
        t = _graph_ms(lambda: [q.aqn_rmsnorm(x, w, EPS, sigma, SEED, RL_STEP, 0, want_f32=False, y_bf16=y)
                               for _ in range(calls)], 10) / calls
        b = norm_bytes(m, h)
        out[f"M={m},H={h}"] = {"us": t * 1e3, "bytes": b, "GB/s": b / (t * 1e-3) / 1e9,
                               "frac": b / (t * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return out


def decode_large_m_leg(dev, ms=(128, 256), copies=4, reps=5):
    """The 32B layer's batched rollout past the ridge (M 128 and 256): the
    same step as the decode layers (norm + q|k|v, o, norm + gate|up, down),
    cold copies, one graph.  Both roofline fractions and T_roof / T."""
    layer = DecodeLayer(dict(LAYER_32B, ms=tuple(ms)), dev, copies=copies)
    out = {}
    for mi, m in enumerate(ms):
        t = _graph_ms(lambda: [layer.step_m(s, m, mi) for s in range(reps)], 3) * 1e-3 / reps
        b = layer.bytes_m(m)
        f = sum(gemm_flops(m, n, k, RANK) for n, k in layer.shapes.values())
        t_roof = max(b / (HBM_PEAK_GBS * 1e9), f / (BF16_MFMA_PEAK_TFLOPS * 1e12))
        out[f"M={m}"] = {"us": t * 1e6, "GB/s": b / t / 1e9, "hbm_frac": b / t / 1e9 / HBM_PEAK_GBS,
                         "tflops": f / t / 1e12, "mfma_frac": f / t / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                         "t_roof_us": t_roof * 1e6, "t_roof_over_t": t_roof / t}
    del layer
    torch.cuda.empty_cache()
    return out


def backward_leg(dev, reps, m=2048):
    """The update phase's backward of the 7B layer's seven projections at M
    tokens (LoRA r = 32 trained, NVFP4 base frozen): dx, dA and dB per
    projection, timed in one graph.  FLOPs per projection: 2 M N K (dy what)
    + 2 M r (N + K) (t and g) + 2 M r K (g A) + 2 M r (K + N) (dA, dB)."""
    layer = make_layer(synth.QWEN25_7B, SEED, dev)
    xs = {name: synth.activation_bf16(m, k, synth.seed_for(SEED, "bx", name), 0.005, device=dev)
          for name, (n, k) in synth.QWEN25_7B.items()}
    dys = {name: synth.activation_bf16(m, n, synth.seed_for(SEED, "bdy", name), 0.0, device=dev)
           for name, (n, k) in synth.QWEN25_7B.items()}
    ws = torch.empty(max(q.w4a16_lora_backward_workspace_size(m, n, k, RANK) for n, k in synth.QWEN25_7B.values()),
                     dtype=torch.uint8, device=dev)
    flops = 0
    for name, (n, k) in synth.QWEN25_7B.items():
        flops += 2 * m * n * k + 2 * m * RANK * (n + k) + 2 * m * RANK * k + 2 * m * RANK * (k + n)

    def run():
        for name in synth.PROJ_ORDER:
            p = layer[name]
            q.w4a16_lora_backward(dys[name], xs[name], p.wq, p.a, p.b, ALPHA / RANK, workspace=ws)

    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    warm_up(g.replay)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del g
    tf = flops / t / 1e12
    return {"workload": f"backward (dx, dA, dB) of the Qwen2.5-7B-shaped layer's 7 projections, M = {m} tokens, "
                        f"LoRA r = {RANK}", "ms": t * 1e3, "tflops": tf, "frac": tf / BF16_MFMA_PEAK_TFLOPS}


def _graph_ms(run, reps):
    """Milliseconds per run(), captured once as a HIP graph and replayed."""
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    # one warm replay, as the step's own timing does: the call-class and
    # per-layer figures are compared with that step and with the rocprofv3
    # traces of the same replays (0.3 s of back-to-back decode replays first
    # made them about 15% slower)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / reps


def update_forward_leg(dev, reps, m=2048):
    """The update phase's forward (the logits pass over the sampled tokens) of
    the 7B layer's seven projections at M tokens, two ways: the fused W4A16 +
    LoRA GEMM, and the unfused route the README's training hints describe
    (each weight dequantized to BF16 by qerl_nvfp4_dequantize, then torch's
    BF16 GEMM and the LoRA products).  The dequantization alone is reported
    as HBM bandwidth: per weight element 0.5 B of codes, 1/16 B of scales and
    2 B of BF16 written."""
    layer = make_layer(synth.QWEN25_7B, SEED, dev)
    xs = {name: synth.activation_bf16(m, k, synth.seed_for(SEED, "fx", name), 0.005, device=dev)
          for name, (n, k) in synth.QWEN25_7B.items()}
    ys = {name: torch.empty((m, n), dtype=torch.bfloat16, device=dev) for name, (n, k) in synth.QWEN25_7B.items()}
    wbf = {name: torch.empty((n, k), dtype=torch.bfloat16, device=dev) for name, (n, k) in synth.QWEN25_7B.items()}
    ws = torch.empty(max(q.w4a16_lora_gemm_workspace_size(m, n, k, RANK) for n, k in synth.QWEN25_7B.values()),
                     dtype=torch.uint8, device=dev)
    lam = ALPHA / RANK

    def fused():
        for name in synth.PROJ_ORDER:
            p = layer[name]
            q.w4a16_lora_gemm(xs[name], p.wq, p.a, p.b, lam, out=ys[name], workspace=ws)

    def dequant():
        for name in synth.PROJ_ORDER:
            q.nvfp4_dequantize(layer[name].wq, out=wbf[name])

    def unfused():
        for name in synth.PROJ_ORDER:
            p, x = layer[name], xs[name]
            q.nvfp4_dequantize(p.wq, out=wbf[name])
            torch.mm(x, wbf[name].t(), out=ys[name])
            ys[name].add_(torch.nn.functional.linear(torch.nn.functional.linear(x, p.a), p.b), alpha=lam)

    t_fused, t_unfused, t_deq = _graph_ms(fused, reps), _graph_ms(unfused, reps), _graph_ms(dequant, reps)
    elems = sum(n * k for n, k in synth.QWEN25_7B.values())
    flops = sum(gemm_flops(m, n, k, RANK) for n, k in synth.QWEN25_7B.values())
    del layer, xs, ys, wbf, ws
    torch.cuda.empty_cache()
    return {"workload": f"forward of the Qwen2.5-7B-shaped layer's 7 projections, M = {m} tokens, LoRA r = {RANK}",
            "fused_w4a16_lora_ms": round(t_fused, 4), "dequant_then_bf16_ms": round(t_unfused, 4),
            "speedup": round(t_unfused / t_fused, 3), "fused_tflops": round(flops / t_fused / 1e9, 1),
            "dequant_ms": round(t_deq, 4), "dequant_gbs": round(elems * (0.5 + 1 / 16 + 2) / t_deq / 1e6, 1)}


E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _dequant_codes(packed):
    """E2M1 values of the codes in packed [N, K/2] (torch, on the GPU)."""
    lut = torch.tensor(list(E2M1_GRID) + [-v for v in E2M1_GRID], dtype=torch.float32, device=packed.device)
    lo, hi = (packed & 15).long(), (packed >> 4).long()
    return torch.stack((lut[lo], lut[hi]), dim=-1).reshape(packed.shape[0], -1)


def quantizer_variants_leg(dev, reps):
    """The quantizer variants the NVFP4 section names: stochastic element
    rounding and MXFP4 (block 32, E8M0 scales), timed on the 32B layer like
    the deterministic quantizer, and the relative L2 error of each format's
    dequantized weights on the 7B layer (the format comparison)."""
    shapes = synth.QWEN25_32B
    ws = torch.empty(q.nvfp4_quantize_workspace_size(1, 16), dtype=torch.uint8, device=dev)
    res = {"workload": "one Qwen2.5-32B-shaped layer (7 tensors, 0.488 G elements); errors on the 7B layer"}
    ws_in, elems = {}, 0
    for name in synth.PROJ_ORDER:
        n, k = shapes[name]
        ws_in[name] = synth.weight_bf16(n, k, seed=synth.seed_for(1005, name), outlier_row_frac=0.001, device=dev)
        elems += n * k
    outs = {name: q.NVFP4Weight(torch.empty((w.shape[0], w.shape[1] // 2), dtype=torch.uint8, device=dev),
                                torch.empty((w.shape[0], w.shape[1] // 16), dtype=torch.uint8, device=dev),
                                torch.empty(1, dtype=torch.float32, device=dev)) for name, w in ws_in.items()}

    def timed(run, bytes_per_elem):
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        return {"ms": t * 1e3, "GB/s": elems * bytes_per_elem / t / 1e9}

    res["nvfp4_stochastic"] = timed(lambda: [q.nvfp4_quantize(ws_in[nm], out=outs[nm], workspace=ws, check_finite=False,
                                                              stochastic_seed=7) for nm in synth.PROJ_ORDER], 4.5625)
    res["mxfp4"] = timed(lambda: [q.mxfp4_quantize(ws_in[nm]) for nm in synth.PROJ_ORDER], 2 + 0.5 + 1 / 32)
    del ws_in, outs
    torch.cuda.empty_cache()
    # format comparison: ||deq(w) - w|| / ||w|| over the 7B layer's weights
    sq = {"nvfp4": 0.0, "nvfp4_stochastic": 0.0, "mxfp4": 0.0}
    ref = 0.0
    for name in synth.PROJ_ORDER:
        n, k = synth.QWEN25_7B[name]
        w = synth.weight_bf16(n, k, seed=synth.seed_for(SEED, name), row_lognormal_sigma=0.5, device=dev)
        wf = w.float()
        ref += float((wf * wf).sum())
        for key, seed in (("nvfp4", None), ("nvfp4_stochastic", 11)):
            wq = q.nvfp4_quantize(w, stochastic_seed=seed)
            sc = wq.scales.view(torch.float8_e4m3fn).float().repeat_interleave(16, dim=1)
            d = _dequant_codes(wq.packed) * sc * wq.tensor_scale
            sq[key] += float(((d - wf) ** 2).sum())
        mp, ms = q.mxfp4_quantize(w)
        sc = torch.exp2(ms.float() - 127.0).repeat_interleave(32, dim=1)
        d = _dequant_codes(mp) * sc
        sq["mxfp4"] += float(((d - wf) ** 2).sum())
        del w, wf
    res["rel_l2_error_7b"] = {key: (v / ref) ** 0.5 for key, v in sq.items()}
    return res


# ---- roofline of the dominant decode kernel --------------------------------
# A decode GEMM call is two launches: the streaming kernel (stream_kernel for
# M <= 16, mfma_unit_kernel for 16 < M <= 256) and finish_kernel, which sums the
# partial tiles and adds the LoRA term.  The unit of the roofline is one call
# (its algorithmic bytes over its duration); the class whose calls take the
# larger share of the step is reported, the other beside it.  Durations come
# from a graph of the step's calls of that class run back to back (cold
# copies rotating), timed with one event pair around the replay.
ROOFLINE_CLASSES = {
    "stream": dict(max_m=16, kernels=("stream_kernel<", "finish_kernel<"),
                   file="decode_stream_kernel_m1_m16.md",
                   sources=("decode.hip", "device_common.h", "qerl_internal.h")),
    "mfma": dict(max_m=64, kernels=("mfma_unit_kernel<", "finish_kernel<", "aqn_rmsnorm_kernel"),
                 file="decode_mfma_unit_kernel_m64.md",
                 sources=("decode.hip", "mfma_tile.h", "device_common.h", "qerl_internal.h", "aqn.hip")),
}


def kernel_sources_sha256(sources):
    """Hash of the kernel's sources with comments and blank lines removed
    (a comment edit does not change the kernel)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "nvfp4_weight_only_quantize_amd", "csrc", f)) as fh:
            for line in fh:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def recorded_traffic(cls):
    """HBM bytes per call from the committed counter summary of the class, or
    None when it is missing or the kernel sources changed since."""
    c = ROOFLINE_CLASSES[cls]
    try:
        with open(os.path.join(ROOT, "profiles", c["file"])) as fh:
            kv = dict(line.strip()[2:].split(": ", 1) for line in fh if line.startswith("- ") and ": " in line)
    except OSError:
        return None
    if kv.get("sources_sha256") != kernel_sources_sha256(c["sources"]):
        return None
    return float(kv["hbm_bytes_per_call"])


def class_calls(layers, cls):
    """(layer, m, mi) of the step whose calls fall in the class."""
    lo = 0 if cls == "stream" else 16
    hi = ROOFLINE_CLASSES[cls]["max_m"]
    return [(L, m, mi) for L in layers for mi, m in enumerate(L.ms) if lo < m <= hi]


def roofline_leg(layers, reps=5, classes=ROOFLINE_CLASSES):
    """Per call class: algorithmic bytes per call over the average call
    duration.  Returns (the class with the larger share of the step, the
    others)."""
    res = {}
    for cls in classes:
        sel = class_calls(layers, cls)
        if not sel:
            continue

        def run(sel=sel):
            for s in range(reps):
                for L, m, mi in sel:
                    L.step_m(1000 + s, m, mi)

        t = _graph_ms(run, 1) * 1e-3
        ncalls = 4 * len(sel) * reps  # four calls per layer step: norm+q|k|v, o, norm+gate|up, down
        b = sum(L.bytes_m(m) for L, m, _ in sel) * reps
        b_call, t_call = b / ncalls, t / ncalls
        achieved = b_call / t_call / 1e9
        res[cls] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(cls),
                    "kernel": f"decode GEMM call ({' + '.join(k.rstrip('<') for k in ROOFLINE_CLASSES[cls]['kernels'])}"
                              f"), M in {sorted({m for _, m, _ in sel})}, layers "
                              f"{sorted({L.cfg['name'] for L, _, _ in sel})}",
                    "calls": ncalls, "avg_call_us": t_call * 1e6, "avg_call_bytes": b_call,
                    "class_step_us": t / reps * 1e6}
    dom = max(res, key=lambda c: res[c]["class_step_us"])
    other = {c: v for c, v in res.items() if c != dom}
    return res[dom], other


def summarize_profile(cls, trace_dir, fetch_dir, write_dir):
    """Print the markdown summary of three rocprofv3 runs of `--calls-only
    CLASS --copy-probe`: kernel statistics of the class's kernels, the
    per-call sum of their durations, and FETCH_SIZE / WRITE_SIZE per call
    scaled by what the counters read for the 256 MiB copy."""
    import csv
    import glob
    c = ROOFLINE_CLASSES[cls]

    def rows(d, pat):
        out = []
        for f in glob.glob(os.path.join(d, "**", pat), recursive=True):
            with open(f) as fh:
                out += list(csv.DictReader(fh))
        return out

    def ours(name):
        return any(k in name for k in c["kernels"])

    stats = rows(trace_dir, "*kernel_stats.csv")
    lines = ["| kernel | calls | average (us) | min (us) | max (us) |", "|---|---:|---:|---:|---:|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:10]:
        nm = r["Name"].replace("qerl::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
        lines.append(f"| `{nm[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    mine = [r for r in stats if ours(r["Name"])]
    calls = sum(int(r["Calls"]) for r in mine if "finish_kernel" in r["Name"])
    tot_ns = sum(float(r["TotalDurationNs"]) for r in mine)
    per_call_us = tot_ns / calls / 1e3 if calls else float("nan")

    def per_call(d, counter):
        vals, copy = 0.0, []
        for r in rows(d, "*counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            if ours(r["Kernel_Name"]):
                vals += float(r["Counter_Value"])
            elif "copyBuffer" in r["Kernel_Name"]:
                copy.append(float(r["Counter_Value"]))
        return vals / max(calls, 1), max(copy) if copy else float("nan")

    f_kib, f_copy = per_call(fetch_dir, "FETCH_SIZE")
    w_kib, w_copy = per_call(write_dir, "WRITE_SIZE")
    copy_kib = 256 * 1024  # the probe copies 256 MiB: that many read and written
    f_scale, w_scale = copy_kib / f_copy, copy_kib / w_copy
    hbm = (f_kib * f_scale + w_kib * w_scale) * 1024
    print("\n".join(lines))
    print()
    print(f"- class: {cls} ({', '.join(k.rstrip('<') for k in c['kernels'])}; {calls} calls)")
    print(f"- kernel_us_per_call: {per_call_us:.3f} (sum of the class's kernel durations / calls)")
    print(f"- fetch_kib_per_call: {f_kib:.1f}")
    print(f"- write_kib_per_call: {w_kib:.1f}")
    print(f"- copy_probe_fetch_kib: {f_copy:.1f} (256 MiB copy; scale {f_scale:.4f})")
    print(f"- copy_probe_write_kib: {w_copy:.1f} (256 MiB copy; scale {w_scale:.4f})")
    print(f"- hbm_bytes_per_call: {hbm:.0f}")
    print(f"- sources_sha256: {kernel_sources_sha256(c['sources'])}")


def summarize_quantizer_profile(trace_dir, fetch_dir, write_dir):
    """Print the markdown summary of three rocprofv3 runs of `--quantizer-only
    --copy-probe` (the 32B layer's seven tensors: amax_kernel then
    encode_kernel each, two-pass timing then one-pass): kernel statistics,
    per-layer durations of each pass, and HBM bytes per layer from
    FETCH_SIZE / WRITE_SIZE scaled by the 256 MiB copy."""
    import csv
    import glob

    def rows(d, pat):
        out = []
        for f in glob.glob(os.path.join(d, "**", pat), recursive=True):
            with open(f) as fh:
                out += list(csv.DictReader(fh))
        return out

    stats = rows(trace_dir, "*kernel_stats.csv")
    lines = ["| kernel | calls | average (us) | min (us) | max (us) |", "|---|---:|---:|---:|---:|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:8]:
        nm = r["Name"].replace("qerl::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
        lines.append(f"| `{nm[:60]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    ours = [r for r in stats if "amax_kernel" in r["Name"] or "encode_kernel<false>" in r["Name"]]
    amax = [r for r in ours if "amax_kernel" in r["Name"]]
    enc = [r for r in ours if "encode_kernel" in r["Name"]]
    layers_amax = sum(int(r["Calls"]) for r in amax) / 7  # two-pass layer quantizations (7 tensors each)
    layers_enc = sum(int(r["Calls"]) for r in enc) / 7    # every layer quantization, both routes
    amax_us = sum(float(r["TotalDurationNs"]) for r in amax) / 1e3 / max(layers_amax, 1)
    enc_us = sum(float(r["TotalDurationNs"]) for r in enc) / 1e3 / max(layers_enc, 1)
    elems = sum(n * k for n, k in synth.QWEN25_32B.values())

    def per_layer(d, counter):
        vals, copy = {"amax": 0.0, "encode": 0.0}, []
        for r in rows(d, "*counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            if "amax_kernel" in r["Kernel_Name"]:
                vals["amax"] += float(r["Counter_Value"])
            elif "encode_kernel<false>" in r["Kernel_Name"]:
                vals["encode"] += float(r["Counter_Value"])
            elif "copyBuffer" in r["Kernel_Name"]:
                copy.append(float(r["Counter_Value"]))
        return vals["amax"] / max(layers_amax, 1), vals["encode"] / max(layers_enc, 1), max(copy) if copy else float("nan")

    fa, fe, f_copy = per_layer(fetch_dir, "FETCH_SIZE")
    wa, we, w_copy = per_layer(write_dir, "WRITE_SIZE")
    copy_kib = 256 * 1024
    fs, ws = copy_kib / f_copy, copy_kib / w_copy
    print("\n".join(lines))
    print()
    print(f"- layer: Qwen2.5-32B-shaped, 7 tensors, {elems / 1e9:.4f} G elements")
    print(f"- amax_us_per_layer: {amax_us:.1f} (pass 1, {layers_amax:.0f} layers)")
    print(f"- encode_us_per_layer: {enc_us:.1f} (pass 2, {layers_enc:.0f} layers)")
    print(f"- two_pass_GB/s: {elems * 4.5625 / ((amax_us + enc_us) * 1e-6) / 1e9:.0f} (4.5625 B per element)")
    print(f"- one_pass_GB/s: {elems * 2.5625 / (enc_us * 1e-6) / 1e9:.0f} (encode only, 2.5625 B per element)")
    print(f"- amax_fetch_kib_per_layer: {fa:.0f}; encode_fetch_kib_per_layer: {fe:.0f}")
    print(f"- amax_write_kib_per_layer: {wa:.0f}; encode_write_kib_per_layer: {we:.0f}")
    print(f"- copy_probe_fetch_kib: {f_copy:.1f} (scale {fs:.4f}); copy_probe_write_kib: {w_copy:.1f} (scale {ws:.4f})")
    print(f"- hbm_bytes_per_layer: amax {fa * fs * 1024:.0f}, encode {(fe * fs + we * ws) * 1024:.0f} "
          f"(algorithmic: amax {2 * elems}, encode {int(2.5625 * elems)})")


def summarize_prefill_profile(trace_dir, fetch_dir, write_dir, mfma_dir):
    """Print the markdown summary of four rocprofv3 runs of `--prefill-only`
    for its dominant launch, prefill_kernel on the fused gate/up GEMM at
    M = 8192 (the largest grid): duration, MFMA busy cycles and HBM bytes."""
    import csv
    import glob

    def rows(d, pat):
        out = []
        for f in glob.glob(os.path.join(d, "**", pat), recursive=True):
            with open(f) as fh:
                out += list(csv.DictReader(fh))
        return out

    def grid(r):
        return int(r.get("Grid_Size", 0) or r.get("Grid_Size_X", 0) or 0)

    tr = [r for r in rows(trace_dir, "*kernel_trace.csv") if "prefill_kernel" in r["Kernel_Name"]]
    top = max(grid(r) for r in tr)
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in tr if grid(r) == top]
    m, (n, k) = 8192, synth.QWEN25_32B["gate"]
    n *= 2
    flops = gemm_flops(m, n, k, 2 * RANK)
    avg = sum(durs) / len(durs)

    def counter(d, name):
        vals = [float(r["Counter_Value"]) for r in rows(d, "*counter_collection.csv")
                if r["Counter_Name"] == name and "prefill_kernel" in r["Kernel_Name"] and grid(r) == top]
        return sum(vals) / max(len(vals), 1), len(vals)

    f_kib, f_n = counter(fetch_dir, "FETCH_SIZE")
    w_kib, w_n = counter(write_dir, "WRITE_SIZE")
    busy, b_n = counter(mfma_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui, _ = counter(mfma_dir, "GRBM_GUI_ACTIVE")  # summed over the 8 XCDs
    cus, xcds = 256, 8  # MI355X
    clock_ghz = gui / xcds / (avg * 1e3)
    print(f"- kernel: prefill_kernel, fused gate/up {n} x {k}, M = {m}, LoRA rank {2 * RANK} "
          f"(grid {top // 256} workgroups, {len(durs)} dispatches)")
    print(f"- average_launch_us: {avg:.1f}")
    print(f"- tflops: {flops / (avg * 1e-6) / 1e12:.1f} ({flops / 1e12:.3f} TFLOP per launch)")
    print(f"- SQ_VALU_MFMA_BUSY_CYCLES: {busy:.4g}; GRBM_GUI_ACTIVE: {gui:.4g} ({b_n} dispatches)")
    print(f"- clock_ghz: {clock_ghz:.2f} (GUI-active cycles per XCD over the traced duration)")
    print(f"- mfma_busy_frac: {busy / (gui / xcds * cus * 4):.3f} (MFMA busy cycles / (GUI-active cycles per XCD x"
          f" {cus} CUs x 4 SIMDs))")
    print(f"- tflops_at_measured_clock_peak_frac: "
          f"{flops / (avg * 1e-6) / (cus * 4 * 1024 * clock_ghz * 1e9):.3f} (1024 BF16 FLOP per SIMD per cycle)")
    print(f"- fetch_kib_per_dispatch: {f_kib:.1f} ({f_n} dispatches; x 2.0 = bytes read, copy-probe scale)")
    print(f"- write_kib_per_dispatch: {w_kib:.1f} ({w_n} dispatches)")
    print(f"- algorithmic_bytes: {n * k * 0.5625 + 2 * m * k + 2 * m * n + 2 * 2 * RANK * (n + k):.0f}")


def decode_breakdown(layers, reps=4):
    """Per layer and M: the step's four calls (norm + q|k|v, o, norm +
    gate|up, down) over `reps` rotating cold copies, replayed as one graph
    120 times; p10 / p50 / p90 of the per-pass time and GB/s at the median."""
    out = {}
    for L in layers:
        for mi, m in enumerate(L.ms):
            p10, p50, p90 = replay_percentiles(lambda L=L, m=m, mi=mi: [L.step_m(s, m, mi) for s in range(reps)])
            b = L.bytes_m(m)
            out[f"{L.cfg['name']} M={m}"] = {"us_p10_p50_p90": [round(p10 / reps, 2), round(p50 / reps, 2),
                                                                round(p90 / reps, 2)],
                                             "bytes": b, "GB/s_p50": round(b / (p50 / reps * 1e-6) / 1e9, 1),
                                             "frac_p50": round(b / (p50 / reps * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--launch", choices=("fused", "streams", "serial"), default="fused",
                    help="q/k/v and gate/up: one multi-segment call each with its norm (fused), side by side "
                         "on side streams after a standalone norm (streams), or one call after another on one "
                         "stream (serial)")
    ap.add_argument("--cpu-budget", type=float, default=30.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-quantizer", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the comparison, rank-sweep, single-layer, norm and large-M legs")
    ap.add_argument("--calls-only", choices=tuple(ROOFLINE_CLASSES),
                    help="only the roofline leg of this call class (for rocprofv3 runs); prints its JSON")
    ap.add_argument("--copy-probe", action="store_true",
                    help="with --calls-only or --quantizer-only: also copy 256 MiB device to device "
                         "(counter scale)")
    ap.add_argument("--summarize", nargs=4, metavar=("CLASS", "TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="print the profile summary of rocprofv3 output directories and exit")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill leg (for rocprofv3 runs); prints its JSON")
    ap.add_argument("--quantizer-only", action="store_true",
                    help="only the one-layer quantizer leg (for rocprofv3 runs); prints its JSON")
    ap.add_argument("--summarize-quantizer", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="print the quantizer profile summary of rocprofv3 output directories and exit")
    ap.add_argument("--summarize-prefill", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "MFMA_DIR"),
                    help="print the prefill profile summary of rocprofv3 output directories and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize_profile(*args.summarize)
        return
    if args.summarize_prefill:
        summarize_prefill_profile(*args.summarize_prefill)
        return
    if args.summarize_quantizer:
        summarize_quantizer_profile(*args.summarize_quantizer)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: there is no multi-GPU path here (pass --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    q.lib()
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_leg(dev, reps=3)}), flush=True)
        return
    if args.quantizer_only:
        q_res = quantizer_leg(dev, reps=3)
        if args.copy_probe:
            src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
        print(json.dumps({"quantizer": q_res}), flush=True)
        return

    log("setting up the decode layers ...")
    layers = [DecodeLayer(LAYER_7B, dev, launch=args.launch), DecodeLayer(LAYER_32B, dev, launch=args.launch)]
    torch.cuda.synchronize()
    if args.calls_only:
        sel = {args.calls_only: ROOFLINE_CLASSES[args.calls_only]}
        roofline, other = roofline_leg(layers, classes=sel)
        if args.copy_probe:
            src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
        print(json.dumps({"roofline": roofline}), flush=True)
        return

    def steps_fn(first, count):
        for s in range(first, first + count):
            for L in layers:
                L.step(s)

    ms_per_step, _graphs = time_graph(steps_fn, args.steps, args.warmup)
    del _graphs
    step_bytes = sum(L.step_bytes() for L in layers)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"decode step {ms_per_step * 1e3:.1f} us, {value:.0f} GB/s")
    p10, p50, p90 = replay_percentiles(lambda: steps_fn(0, 4))
    roofline, roofline_other = roofline_leg(layers)
    breakdown = decode_breakdown(layers)
    log("parity against the oracle ...")
    parity = check_decode_parity(layers)
    result = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode of a Qwen2.5-7B-shaped layer at M in {1, 8, 64} and a Qwen2.5-32B-shaped "
                               "layer at M in {16, 64}: AQN RMSNorm + q|k|v, o, AQN RMSNorm + gate|up, down, "
                               "NVFP4 W4A16 + LoRA r32 (alpha 64) on all seven projections",
                   "layers": [{"name": L.cfg["name"], "hidden": L.cfg["hidden"], "intermediate": L.cfg["inter"],
                               "decode_m": list(L.ms), "cold_weight_copies": len(L.copies)} for L in layers],
                   "lora_rank": RANK, "hip_graph": True, "launch": args.launch, "step_bytes": step_bytes},
        "frac_of_hbm_peak": value / HBM_PEAK_GBS,
        "step_us_p10_p50_p90": [round(p10 / 4, 2), round(p50 / 4, 2), round(p90 / 4, 2)],
        "roofline": roofline,
        "roofline_secondary": roofline_other,
        "decode_breakdown": breakdown,
        "parity_rel_l2_smallest_m": parity,
    }
    if not args.no_extras:
        log("BF16 + LoRA comparison and LoRA rank sweep ...")
        result["bf16_lora_compare_7b"] = bf16_lora_leg(layers[0])
        result["lora_rank_sweep_7b"] = lora_rank_leg(layers[0])
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline ...")
        cpu = cpu_baseline(layers, args.cpu_budget)
    del layers
    torch.cuda.empty_cache()
    if not args.no_extras:
        log("32B layer at M 128 and 256 ...")
        result["decode_32b_large_m"] = decode_large_m_leg(dev)
        log("single 2048 x 2048 layer ...")
        result["single_layer_2048"] = single_layer_leg(dev)
        log("AQN RMSNorm alone ...")
        result["aqn_rmsnorm"] = aqn_leg(dev)
    if not args.no_prefill:
        log("prefill leg ...")
        result["prefill"] = prefill_leg(dev, reps=3)
    if not args.no_quantizer:
        log("quantizer legs ...")
        result["quantizer"] = {"layer_32b": quantizer_leg(dev, reps=3),
                               "model_32b": model_quantizer_leg(dev),
                               "variants": quantizer_variants_leg(dev, reps=3)}
    if not args.no_backward:
        log("update-phase forward: fused W4A16 + LoRA against dequantize + BF16 GEMM ...")
        result["update_forward"] = update_forward_leg(dev, reps=3)
        log("backward leg ...")
        result["backward"] = backward_leg(dev, reps=3)
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
