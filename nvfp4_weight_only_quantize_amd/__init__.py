"""MI355X-native NVFP4 weight-only (W4A16) + LoRA linear layer of QeRL.

Thin Python binding over ``libqerl.so`` (C ABI in ``include/qerl.h``): it
only checks tensor metadata, allocates outputs/workspaces with PyTorch and
passes raw device pointers and the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no Python or CPU
fallback -- calls fail loudly when the library is not built.

Functions (same names as the C entry points, without the ``qerl_`` prefix):

* :func:`nvfp4_quantize`  -- BF16 [N, K] -> :class:`NVFP4Weight`
* :func:`w4a16_lora_gemm` -- y = x deq(W)^T + lora_scale (x A^T) B^T
* :func:`aqn_rmsnorm`     -- RMSNorm with the AQN noisy scale vector
* :func:`aqn_sigma`       -- exponential sigma schedule (host)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqerl.so")

QERL_OK = 0
STATUS_NAMES = {0: "QERL_OK", 1: "QERL_ERR_NULL", 2: "QERL_ERR_SHAPE", 3: "QERL_ERR_ALIGN",
                4: "QERL_ERR_ARG", 5: "QERL_ERR_WORKSPACE", 6: "QERL_ERR_HIP"}
SCALE_ROUND_UP = 0
SCALE_RNE = 1
MAX_LORA_RANK = 128
MAX_NORM_WIDTH = 16384

_lib = None


class QerlError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libqerl.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m nvfp4_weight_only_quantize_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32, u32, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float,
                                      ctypes.c_size_t)
    L.qerl_nvfp4_quantize_workspace_size.argtypes = [i64, i64]
    L.qerl_nvfp4_quantize_workspace_size.restype = sz
    L.qerl_nvfp4_quantize.argtypes = [P, i64, i64, i64, P, P, P, P, u32, P, sz, P]
    L.qerl_nvfp4_quantize.restype = ctypes.c_int
    L.qerl_nvfp4_quantize_stochastic.argtypes = [P, i64, i64, i64, P, P, P, P, u32, u64, P, sz, P]
    L.qerl_nvfp4_quantize_stochastic.restype = ctypes.c_int
    L.qerl_mxfp4_quantize.argtypes = [P, i64, i64, i64, P, P, P]
    L.qerl_mxfp4_quantize.restype = ctypes.c_int
    L.qerl_nvfp4_dequantize.argtypes = [P, P, P, i64, i64, P, i64, P]
    L.qerl_nvfp4_dequantize.restype = ctypes.c_int
    L.qerl_w4a16_lora_gemm_workspace_size.argtypes = [i64, i64, i64, i32]
    L.qerl_w4a16_lora_gemm_workspace_size.restype = sz
    L.qerl_w4a16_lora_gemm.argtypes = [P, i64, i64, i64, P, P, P, i64, P, P, i32, f32, P, i64,
                                       P, sz, P]
    L.qerl_w4a16_lora_gemm.restype = ctypes.c_int
    L.qerl_w4a16_lora_gemm_noalloc.argtypes = [P, i64, i64, i64, P, P, P, i64, P, P, i32, f32, P, i64, P]
    L.qerl_w4a16_lora_gemm_noalloc.restype = ctypes.c_int
    L.qerl_w4a16_lora_gemm_multi_workspace_size.argtypes = [i64, i64, ctypes.POINTER(GemmSegment), i32]
    L.qerl_w4a16_lora_gemm_multi_workspace_size.restype = sz
    L.qerl_w4a16_lora_gemm_multi.argtypes = [P, i64, i64, i64, ctypes.POINTER(GemmSegment), i32, P, sz, P]
    L.qerl_w4a16_lora_gemm_multi.restype = ctypes.c_int
    L.qerl_rmsnorm_w4a16_lora_gemm_multi_workspace_size.argtypes = [i64, i64, ctypes.POINTER(GemmSegment), i32]
    L.qerl_rmsnorm_w4a16_lora_gemm_multi_workspace_size.restype = sz
    L.qerl_rmsnorm_w4a16_lora_gemm_multi.argtypes = [P, i64, i64, i64, P, f32, ctypes.POINTER(GemmSegment), i32,
                                                     P, sz, P]
    L.qerl_rmsnorm_w4a16_lora_gemm_multi.restype = ctypes.c_int
    L.qerl_aqn_noisy_weight.argtypes = [P, i64, f32, u64, u64, u32, P, P]
    L.qerl_aqn_noisy_weight.restype = ctypes.c_int
    L.qerl_w4a16_lora_backward_workspace_size.argtypes = [i64, i64, i64, i32]
    L.qerl_w4a16_lora_backward_workspace_size.restype = sz
    L.qerl_w4a16_lora_backward.argtypes = [P, i64, i64, i64, P, i64, i64, P, P, P, P, P, i32, f32, P, i64, P, P,
                                           P, sz, P]
    L.qerl_w4a16_lora_backward.restype = ctypes.c_int
    L.qerl_aqn_sigma.argtypes = [i32, i32, f32, f32]
    L.qerl_aqn_sigma.restype = f32
    L.qerl_aqn_rmsnorm.argtypes = [P, i64, i64, i64, P, f32, f32, u64, u64, u32, P, P, i64, P, P]
    L.qerl_aqn_rmsnorm.restype = ctypes.c_int
    L.qerl_status_string.argtypes = [ctypes.c_int]
    L.qerl_status_string.restype = ctypes.c_char_p
    L.qerl_last_error.argtypes = []
    L.qerl_last_error.restype = ctypes.c_char_p
    L.qerl_last_hip_error.argtypes = []
    L.qerl_last_hip_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != QERL_OK:
        raise QerlError(status, lib().qerl_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")


def _rows(t: torch.Tensor, name: str) -> int:
    """Leading dimension of a 2-D tensor whose rows are contiguous."""
    if t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous")
    return t.stride(0) if t.size(0) > 1 else t.size(1)


@dataclass
class NVFP4Weight:
    """NVFP4 tensor: packed E2M1 codes [N, K/2] (even element in the low nibble),
    E4M3 block scales [N, K/16] and the FP32 tensor scale [1], all on the GPU."""
    packed: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor

    @property
    def shape(self):
        return (self.packed.size(0), self.packed.size(1) * 2)

    @property
    def nbytes(self) -> int:
        return self.packed.numel() + self.scales.numel() + 4


def _need_wq(wq: NVFP4Weight, device):
    """An NVFP4 weight the kernels can read: contiguous uint8 packed [N, K/2]
    and scales [N, K/16] and one FP32 tensor scale, on `device`."""
    _need(wq.packed, "packed", torch.uint8, 2, device)
    _need(wq.scales, "scales", torch.uint8, 2, device)
    _need(wq.tensor_scale, "tensor_scale", torch.float32, None, device)
    n, k = wq.shape
    if tuple(wq.scales.shape) != (n, k // 16) or wq.tensor_scale.numel() != 1:
        raise ValueError("NVFP4 weight: scales must be [N, K/16] and tensor_scale one element")
    if not (wq.packed.is_contiguous() and wq.scales.is_contiguous()):
        raise ValueError("NVFP4 weight: packed and scales must be contiguous")


# --------------------------------------------------------------- quantizer --
def nvfp4_quantize_workspace_size(n: int, k: int) -> int:
    return int(lib().qerl_nvfp4_quantize_workspace_size(n, k))


def nvfp4_quantize(w: torch.Tensor, flags: int = SCALE_ROUND_UP, tensor_scale_in=None,
                   out: NVFP4Weight | None = None, workspace: torch.Tensor | None = None,
                   stream=None, check_finite: bool = True, stochastic_seed: int | None = None) -> NVFP4Weight:
    """Quantize a BF16 [N, K] GPU tensor to NVFP4 (K % 16 == 0).

    ``check_finite`` synchronizes and raises if the tensor held a NaN/Inf (the
    library reports it in-band as a NaN tensor scale).  ``stochastic_seed``:
    stochastic element rounding with that seed (qerl_nvfp4_quantize_stochastic)."""
    _need(w, "w", torch.bfloat16, 2)
    n, k = w.shape
    ldw = _rows(w, "w")
    dev = w.device
    if out is None:
        out = NVFP4Weight(torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
                          torch.empty((n, max(k // 16, 0)), dtype=torch.uint8, device=dev),
                          torch.empty(1, dtype=torch.float32, device=dev))
    if tensor_scale_in is not None:
        _need(tensor_scale_in, "tensor_scale_in", torch.float32, device=dev)
    if workspace is None and tensor_scale_in is None:
        workspace = torch.empty(nvfp4_quantize_workspace_size(n, k), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if stochastic_seed is None:
        _check(lib().qerl_nvfp4_quantize(_ptr(w), n, k, ldw, _ptr(out.packed), _ptr(out.scales),
                                         _ptr(out.tensor_scale), _ptr(tensor_scale_in), int(flags),
                                         _ptr(workspace), ws_bytes, _stream(stream, dev)))
    else:
        _check(lib().qerl_nvfp4_quantize_stochastic(_ptr(w), n, k, ldw, _ptr(out.packed), _ptr(out.scales),
                                                    _ptr(out.tensor_scale), _ptr(tensor_scale_in), int(flags),
                                                    int(stochastic_seed) & (2 ** 64 - 1), _ptr(workspace),
                                                    ws_bytes, _stream(stream, dev)))
    if check_finite and not torch.isfinite(out.tensor_scale).all().item():
        raise QerlError(4, "weight tensor holds a NaN or Inf (tensor scale is NaN)")
    return out


def mxfp4_quantize(w: torch.Tensor, stream=None):
    """BF16 [N, K] GPU tensor (K % 32 == 0) -> (packed u8 [N, K/2], E8M0 scales u8 [N, K/32])."""
    _need(w, "w", torch.bfloat16, 2)
    n, k = w.shape
    dev = w.device
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((n, max(k // 32, 0)), dtype=torch.uint8, device=dev)
    _check(lib().qerl_mxfp4_quantize(_ptr(w), n, k, _rows(w, "w"), _ptr(packed), _ptr(scales),
                                     _stream(stream, dev)))
    return packed, scales


def nvfp4_dequantize(wq: NVFP4Weight, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """BF16 [N, K] = e2m1 x e4m3 x s_t of an NVFP4 weight, rounded once to BF16."""
    n, k = wq.shape
    dev = wq.packed.device
    _need_wq(wq, dev)
    if out is None:
        out = torch.empty((n, k), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (n, k):
        raise ValueError(f"out shape {tuple(out.shape)} != {(n, k)}")
    _check(lib().qerl_nvfp4_dequantize(_ptr(wq.packed), _ptr(wq.scales), _ptr(wq.tensor_scale), n, k, _ptr(out),
                                       _rows(out, "out"), _stream(stream, dev)))
    return out


# --------------------------------------------------------- W4A16 + LoRA ----
def w4a16_lora_gemm_workspace_size(m: int, n: int, k: int, r: int) -> int:
    return int(lib().qerl_w4a16_lora_gemm_workspace_size(m, n, k, r))


def _gemm_operands(x, wq, lora_a, lora_b, out):
    """Checks of the single-projection GEMM's tensors; returns (m, n, k, r, out)."""
    _need(x, "x", torch.bfloat16, 2)
    dev = x.device
    m, k = x.shape
    _need_wq(wq, dev)
    n, kw = wq.shape
    if kw != k:
        raise ValueError(f"x has K={k} but the weight has K={kw}")
    r = 0
    if lora_a is not None or lora_b is not None:
        _need(lora_a, "lora_a", torch.bfloat16, 2, dev)
        _need(lora_b, "lora_b", torch.bfloat16, 2, dev)
        r = lora_a.size(0)
        if tuple(lora_a.shape) != (r, k) or tuple(lora_b.shape) != (n, r):
            raise ValueError("LoRA shapes must be A [r, K] and B [N, r]")
        if not (lora_a.is_contiguous() and lora_b.is_contiguous()):
            raise ValueError("LoRA matrices must be contiguous")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, 2, dev)
    if tuple(out.shape) != (m, n):
        raise ValueError("out must be [M, N]")
    return m, n, k, r, out


def w4a16_lora_gemm(x: torch.Tensor, wq: NVFP4Weight, lora_a: torch.Tensor | None = None,
                    lora_b: torch.Tensor | None = None, lora_scale: float = 0.0,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """y [M, N] (BF16) = x [M, K] deq(W)^T + lora_scale (x A^T) B^T.

    A caller-provided ``workspace`` (uint8, at least the size query) holds
    partial sums only: any contents, reusable by any sequence of calls on one
    stream."""
    m, n, k, r, out = _gemm_operands(x, wq, lora_a, lora_b, out)
    dev = x.device
    need = w4a16_lora_gemm_workspace_size(m, n, k, r)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qerl_w4a16_lora_gemm(
        _ptr(x), m, k, _rows(x, "x"), _ptr(wq.packed), _ptr(wq.scales), _ptr(wq.tensor_scale), n,
        _ptr(lora_a), _ptr(lora_b), r, float(lora_scale), _ptr(out), _rows(out, "out"),
        _ptr(workspace), ws_bytes, _stream(stream, dev)))
    return out


NOALLOC_SCRATCH_BYTES = 48 << 20  # QERL_NOALLOC_SCRATCH_BYTES


def w4a16_lora_gemm_noalloc(x: torch.Tensor, wq: NVFP4Weight, lora_a: torch.Tensor | None,
                            lora_b: torch.Tensor | None, lora_scale: float, out: torch.Tensor,
                            stream=None) -> torch.Tensor:
    """The layer of w4a16_lora_gemm through qerl_w4a16_lora_gemm_noalloc: no
    workspace, the partial sums go to the library's static per-device scratch
    (sizes whose workspace query exceeds NOALLOC_SCRATCH_BYTES are rejected).
    ``out`` is required so that nothing is allocated here either.  Calls that
    overlap in time on one device race on the shared scratch."""
    if out is None:
        raise ValueError("out is required")
    m, n, k, r, out = _gemm_operands(x, wq, lora_a, lora_b, out)
    _check(lib().qerl_w4a16_lora_gemm_noalloc(
        _ptr(x), m, k, _rows(x, "x"), _ptr(wq.packed), _ptr(wq.scales), _ptr(wq.tensor_scale), n,
        _ptr(lora_a), _ptr(lora_b), r, float(lora_scale), _ptr(out), _rows(out, "out"),
        _stream(stream, x.device)))
    return out


class GemmSegment(ctypes.Structure):
    """qerl_gemm_segment of include/qerl.h."""
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("tensor_scale", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("lora_a_bf16", ctypes.c_void_p), ("lora_b_bf16", ctypes.c_void_p),
                ("r", ctypes.c_int32), ("lora_scale", ctypes.c_float), ("y_bf16", ctypes.c_void_p),
                ("ldy", ctypes.c_int64)]


MAX_SEGMENTS = 4  # QERL_MAX_SEGMENTS


def _segments(x, segments, outs):
    """ctypes array of the segments (wq, lora_a, lora_b, lora_scale) with outputs."""
    dev = x.device
    m, k = x.shape
    arr = (GemmSegment * len(segments))()
    for i, ((wq, a, b, lam), out) in enumerate(zip(segments, outs)):
        _need_wq(wq, dev)
        n, kw = wq.shape
        if kw != k:
            raise ValueError(f"segment {i}: x has K={k} but the weight has K={kw}")
        r = 0
        if a is not None or b is not None:
            _need(a, "lora_a", torch.bfloat16, 2, dev)
            _need(b, "lora_b", torch.bfloat16, 2, dev)
            r = a.size(0)
            if tuple(a.shape) != (r, k) or tuple(b.shape) != (n, r) or not (a.is_contiguous() and b.is_contiguous()):
                raise ValueError(f"segment {i}: LoRA must be contiguous A [r, K] and B [N, r]")
        _need(out, "out", torch.bfloat16, 2, dev)
        if tuple(out.shape) != (m, n):
            raise ValueError(f"segment {i}: out must be [M, N]")
        arr[i] = GemmSegment(_ptr(wq.packed), _ptr(wq.scales), _ptr(wq.tensor_scale), n, _ptr(a), _ptr(b), r,
                             float(lam), _ptr(out), _rows(out, "out"))
    return arr


def w4a16_lora_gemm_multi_workspace_size(m: int, k: int, shapes) -> int:
    """shapes: (n, r) per segment."""
    arr = (GemmSegment * len(shapes))()
    for i, (n, r) in enumerate(shapes):
        arr[i].n, arr[i].r = int(n), int(r)
    return int(lib().qerl_w4a16_lora_gemm_multi_workspace_size(m, k, arr, len(shapes)))


def w4a16_lora_gemm_multi(x: torch.Tensor, segments, outs=None, workspace: torch.Tensor | None = None,
                          stream=None):
    """Several projections of x in one call: segments is a list of
    (wq, lora_a, lora_b, lora_scale) (LoRA None for none); returns the outputs
    (given in ``outs`` or allocated).  For M <= 256 they share one launch."""
    _need(x, "x", torch.bfloat16, 2)
    if not 1 <= len(segments) <= MAX_SEGMENTS:
        raise ValueError(f"1 to {MAX_SEGMENTS} segments")
    dev = x.device
    m, k = x.shape
    if outs is None:
        outs = [torch.empty((m, wq.shape[0]), dtype=torch.bfloat16, device=dev) for wq, *_ in segments]
    arr = _segments(x, segments, outs)
    need = int(lib().qerl_w4a16_lora_gemm_multi_workspace_size(m, k, arr, len(segments)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qerl_w4a16_lora_gemm_multi(_ptr(x), m, k, _rows(x, "x"), arr, len(segments), _ptr(workspace),
                                            ws_bytes, _stream(stream, dev)))
    return outs


def rmsnorm_w4a16_lora_gemm_multi_workspace_size(m: int, k: int, shapes) -> int:
    """shapes: (n, r) per segment."""
    arr = (GemmSegment * len(shapes))()
    for i, (n, r) in enumerate(shapes):
        arr[i].n, arr[i].r = int(n), int(r)
    return int(lib().qerl_rmsnorm_w4a16_lora_gemm_multi_workspace_size(m, k, arr, len(shapes)))


def rmsnorm_w4a16_lora_gemm_multi(x: torch.Tensor, norm_weight: torch.Tensor, eps: float, segments, outs=None,
                                  workspace: torch.Tensor | None = None, stream=None):
    """RMSNorm of x with scale vector norm_weight (FP32 [K]; the AQN noisy
    weight) and then the projections of w4a16_lora_gemm_multi on the normed
    rows, in one call (for M <= 16 and K % 32 == 0 one launch)."""
    _need(x, "x", torch.bfloat16, 2)
    if not 1 <= len(segments) <= MAX_SEGMENTS:
        raise ValueError(f"1 to {MAX_SEGMENTS} segments")
    dev = x.device
    m, k = x.shape
    _need(norm_weight, "norm_weight", torch.float32, 1, dev)
    if norm_weight.numel() != k or not norm_weight.is_contiguous():
        raise ValueError("norm_weight must be a contiguous [K] tensor")
    if outs is None:
        outs = [torch.empty((m, wq.shape[0]), dtype=torch.bfloat16, device=dev) for wq, *_ in segments]
    arr = _segments(x, segments, outs)
    need = int(lib().qerl_rmsnorm_w4a16_lora_gemm_multi_workspace_size(m, k, arr, len(segments)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qerl_rmsnorm_w4a16_lora_gemm_multi(_ptr(x), m, k, _rows(x, "x"), _ptr(norm_weight), float(eps), arr,
                                                    len(segments), _ptr(workspace), ws_bytes, _stream(stream, dev)))
    return outs


def w4a16_lora_backward_workspace_size(m: int, n: int, k: int, r: int) -> int:
    return int(lib().qerl_w4a16_lora_backward_workspace_size(m, n, k, r))


def w4a16_lora_backward(dy: torch.Tensor, x: torch.Tensor, wq: NVFP4Weight, lora_a: torch.Tensor | None = None,
                        lora_b: torch.Tensor | None = None, lora_scale: float = 0.0, want_dx: bool = True,
                        want_lora: bool = True, workspace: torch.Tensor | None = None, stream=None):
    """Gradients of the layer for upstream dy [M, N]: returns (dx BF16 [M, K] or
    None, dA FP32 [r, K] or None, dB FP32 [N, r] or None)."""
    _need(dy, "dy", torch.bfloat16, 2)
    dev = dy.device
    _need(x, "x", torch.bfloat16, 2, dev)
    m, n = dy.shape
    k = x.shape[1]
    _need_wq(wq, dev)
    if x.shape[0] != m or tuple(wq.shape) != (n, k):
        raise ValueError("dy [M, N], x [M, K] and the weight [N, K] must agree")
    r = 0
    if lora_a is not None or lora_b is not None:
        _need(lora_a, "lora_a", torch.bfloat16, 2, dev)
        _need(lora_b, "lora_b", torch.bfloat16, 2, dev)
        r = lora_a.size(0)
        if tuple(lora_a.shape) != (r, k) or tuple(lora_b.shape) != (n, r):
            raise ValueError("LoRA must be A [r, K] and B [N, r]")
        # the kernels index A and B with row strides K and r
        if not (lora_a.is_contiguous() and lora_b.is_contiguous()):
            raise ValueError("LoRA matrices must be contiguous")
    dx = torch.empty((m, k), dtype=torch.bfloat16, device=dev) if want_dx else None
    da = torch.empty((r, k), dtype=torch.float32, device=dev) if (want_lora and r) else None
    db = torch.empty((n, r), dtype=torch.float32, device=dev) if (want_lora and r) else None
    need = w4a16_lora_backward_workspace_size(m, n, k, r)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().qerl_w4a16_lora_backward(_ptr(dy), m, n, _rows(dy, "dy"), _ptr(x), k, _rows(x, "x"),
                                          _ptr(wq.packed), _ptr(wq.scales), _ptr(wq.tensor_scale), _ptr(lora_a),
                                          _ptr(lora_b), r, float(lora_scale), _ptr(dx), k, _ptr(da), _ptr(db),
                                          _ptr(workspace), ws_bytes, _stream(stream, dev)))
    return dx, da, db


# -------------------------------------------------------------------- AQN --
def aqn_noisy_weight(weight: torch.Tensor, sigma: float, seed: int = 0, step: int = 0, layer_id: int = 0,
                     out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """w + sigma z, the scale vector aqn_rmsnorm multiplies by for the same
    (seed, step, layer_id)."""
    _need(weight, "weight", torch.float32, 1)
    dev = weight.device
    if not weight.is_contiguous():
        raise ValueError("weight must be contiguous")
    if out is None:
        out = torch.empty_like(weight)
    _need(out, "out", torch.float32, 1, dev)
    if out.numel() != weight.numel() or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like weight")
    _check(lib().qerl_aqn_noisy_weight(_ptr(weight), weight.numel(), float(sigma), int(seed) & (2 ** 64 - 1),
                                       int(step) & (2 ** 64 - 1), int(layer_id) & 0xFFFFFFFF, _ptr(out),
                                       _stream(stream, dev)))
    return out

def aqn_sigma(stage: int, num_stages: int, sigma_start: float, sigma_end: float) -> float:
    return float(lib().qerl_aqn_sigma(int(stage), int(num_stages), float(sigma_start),
                                      float(sigma_end)))


def aqn_rmsnorm(x: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6, sigma: float = 0.0,
                seed: int = 0, step: int = 0, layer_id: int = 0, want_f32: bool = True,
                want_bf16: bool = False, y_f32: torch.Tensor | None = None,
                y_bf16: torch.Tensor | None = None, noisy_weight_out: torch.Tensor | None = None,
                stream=None):
    """Returns (y_f32 or None, y_bf16 or None) for x [M, H] BF16 and weight [H] FP32."""
    _need(x, "x", torch.bfloat16, 2)
    dev = x.device
    _need(weight, "weight", torch.float32, 1, dev)
    m, h = x.shape
    if weight.numel() != h or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous [H] tensor")
    if y_f32 is None and want_f32:
        y_f32 = torch.empty((m, h), dtype=torch.float32, device=dev)
    if y_bf16 is None and want_bf16:
        y_bf16 = torch.empty((m, h), dtype=torch.bfloat16, device=dev)
    ldy = None
    for t, nm, dt in ((y_f32, "y_f32", torch.float32), (y_bf16, "y_bf16", torch.bfloat16)):
        if t is not None:
            _need(t, nm, dt, 2, dev)
            if tuple(t.shape) != (m, h):
                raise ValueError(f"{nm} must be [M, H]")
            ld = _rows(t, nm)
            if ldy is not None and ld != ldy:
                raise ValueError("y_f32 and y_bf16 must share a row stride")
            ldy = ld
    if ldy is None:
        raise ValueError("ask for y_f32, y_bf16 or both")
    if noisy_weight_out is not None:
        _need(noisy_weight_out, "noisy_weight_out", torch.float32, 1, dev)
        if noisy_weight_out.numel() != h:
            raise ValueError("noisy_weight_out must be [H]")
    _check(lib().qerl_aqn_rmsnorm(_ptr(x), m, h, _rows(x, "x"), _ptr(weight), float(eps),
                                  float(sigma), int(seed) & (2 ** 64 - 1), int(step) & (2 ** 64 - 1),
                                  int(layer_id) & 0xFFFFFFFF, _ptr(y_f32), _ptr(y_bf16), ldy,
                                  _ptr(noisy_weight_out), _stream(stream, dev)))
    return y_f32, y_bf16
