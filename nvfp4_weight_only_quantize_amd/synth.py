"""Seeded synthetic inputs shaped like the Qwen2.5 layers of the QeRL pages.

This module holds no arithmetic of the method (no quantization, no matmul,
no normalization, no noise stream of AQN).  It only draws random tensors with
the stated distributions, so that the HIP path and the CPU oracle can be fed
the same bits.  Every tensor is drawn in float32 by a ``torch.Generator``
seeded from ``(master seed, tensor id...)`` and rounded to BF16 once.

Shapes: the pages name Qwen2.5 3B-32B models ("Paper 2510.11696 -- QeRL:
Beyond Efficiency", "Summary"; the README's quantize_nvfp4.py invocations).
The projection shapes below are the public Qwen2.5-7B and -32B layouts
(hidden 3584 / 5120, intermediate 18944 / 27648, 4 / 8 KV heads of dim 128).
"""
from __future__ import annotations

import torch

_MASK64 = (1 << 64) - 1

# (N, K) of each projection: y = x W^T with W [N, K]
QWEN25_7B = {
    "q": (3584, 3584), "k": (512, 3584), "v": (512, 3584), "o": (3584, 3584),
    "gate": (18944, 3584), "up": (18944, 3584), "down": (3584, 18944),
}
QWEN25_32B = {
    "q": (5120, 5120), "k": (1024, 5120), "v": (1024, 5120), "o": (5120, 5120),
    "gate": (27648, 5120), "up": (27648, 5120), "down": (5120, 27648),
}
PROJ_ORDER = ("q", "k", "v", "o", "gate", "up", "down")


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _MASK64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def seed_for(master: int, *ids) -> int:
    """Derive a 63-bit generator seed from a master seed and tensor ids."""
    h = _splitmix64(int(master) & _MASK64)
    for i in ids:
        if isinstance(i, str):
            i = int.from_bytes(i.encode()[:8].ljust(8, b"\0"), "little")
        h = _splitmix64(h ^ (int(i) & _MASK64))
    return h & 0x7FFF_FFFF_FFFF_FFFF


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_f32(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * float(std)


def weight_bf16(n: int, k: int, seed: int, std: float = 0.02, row_lognormal_sigma: float = 0.0,
                outlier_row_frac: float = 0.0, outlier_scale: float = 20.0,
                device="cpu") -> torch.Tensor:
    """W [N, K] ~ N(0, std^2), optionally times a per-row log-normal factor
    exp(N(0, sigma^2)) and with round(frac * N) outlier rows scaled up."""
    w = normal_f32((n, k), std, seed_for(seed, "w"), device)
    if row_lognormal_sigma > 0.0:
        f = torch.exp(normal_f32((n, 1), row_lognormal_sigma, seed_for(seed, "rowscale"), device))
        w = w * f
    n_out = int(round(outlier_row_frac * n))
    if n_out > 0:
        g = _gen(seed_for(seed, "outrows"), "cpu")
        rows = torch.randperm(n, generator=g)[:n_out].to(device)
        w[rows] = w[rows] * float(outlier_scale)
    return w.to(torch.bfloat16)


def activation_bf16(m: int, k: int, seed: int, outlier_col_frac: float = 0.0,
                    outlier_scale: float = 20.0, device="cpu") -> torch.Tensor:
    """x [M, K] ~ N(0, 1) with round(frac * K) outlier channels (columns shared
    by every row, picked by a seeded permutation) scaled by outlier_scale."""
    x = normal_f32((m, k), 1.0, seed_for(seed, "x"), device)
    n_out = int(round(outlier_col_frac * k))
    if n_out > 0:
        g = _gen(seed_for(seed, "outcols"), "cpu")
        cols = torch.randperm(k, generator=g)[:n_out].to(device)
        x[:, cols] = x[:, cols] * float(outlier_scale)
    return x.to(torch.bfloat16)


def lora_bf16(n: int, k: int, r: int, seed: int, b_std: float = 0.02, device="cpu"):
    """A [r, K] ~ N(0, 1/K) (std K^-1/2), B [N, r] ~ N(0, b_std^2)."""
    a = normal_f32((r, k), k ** -0.5, seed_for(seed, "A"), device).to(torch.bfloat16)
    b = normal_f32((n, r), b_std, seed_for(seed, "B"), device).to(torch.bfloat16)
    return a, b


def norm_weight_f32(h: int, seed: int, device="cpu") -> torch.Tensor:
    """RMSNorm weight w_c = 1 + 0.1 N(0, 1), FP32."""
    return 1.0 + normal_f32((h,), 0.1, seed_for(seed, "normw"), device)


def bf16_bits(t: torch.Tensor):
    """BF16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")


def bits_to_bf16(a) -> torch.Tensor:
    """numpy uint16 bit patterns -> BF16 CPU tensor."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
