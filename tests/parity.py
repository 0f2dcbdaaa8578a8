"""Helpers shared by the GPU parity tests: move seeded inputs to the GPU,
bring results back as bit patterns, and measure errors against the oracle.

Tolerances (float parts) are the contract's:
* GEMM (FP32 accumulation, BF16 output): relative L2 <= 5e-3 and
  max |y - y_ref| <= 1e-2 * max |y_ref|;
* AQN RMSNorm FP32 output: relative error <= 1e-5 per element;
and the quantizer is compared bit for bit.
"""
import numpy as np
import torch

GEMM_REL_L2 = 5e-3
GEMM_MAX_REL = 1e-2
AQN_REL = 1e-5


def dev():
    return torch.device("cuda", 0)


def bits_to_gpu(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def gpu_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def gemm_errors(y: np.ndarray, ref: np.ndarray):
    """(relative L2, max abs error / max |ref|)"""
    d = y - ref
    nref = np.linalg.norm(ref)
    mref = np.abs(ref).max()
    rel = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    mx = np.abs(d).max() / mref if mref > 0 else np.abs(d).max()
    return float(rel), float(mx)


def assert_gemm_close(y: np.ndarray, ref: np.ndarray, what: str = ""):
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    rel, mx = gemm_errors(y, ref)
    assert rel <= GEMM_REL_L2 and mx <= GEMM_MAX_REL, f"{what}: rel_l2={rel:.3e} max={mx:.3e}"
    return rel, mx
