"""The C ABI: libqerl.so loads, exports every function include/qerl.h
declares, and rejects bad arguments on the host before anything is launched
(no call here reaches the GPU)."""
import ctypes
import math
import os
import re

import pytest

import oracle
import nvfp4_weight_only_quantize_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qerl.h")

pytestmark = pytest.mark.skipif(not os.path.exists(q.LIB_PATH), reason="libqerl.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qerl_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = _declared_functions()
    assert {"qerl_nvfp4_quantize", "qerl_w4a16_lora_gemm", "qerl_aqn_rmsnorm"} <= set(names)
    L = ctypes.CDLL(q.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_status_strings():
    L = q.lib()
    for s in range(7):
        assert L.qerl_status_string(s)
    assert L.qerl_status_string(99) == b"unknown status"


def test_sigma_schedule_matches_oracle():
    for k in range(10):
        got = q.aqn_sigma(k, 10, 1e-2, 5e-4)
        want = oracle.aqn_sigma(k, 10, float(ctypes.c_float(1e-2).value), float(ctypes.c_float(5e-4).value))
        assert abs(got - want) <= 1e-7 * want
    assert q.aqn_sigma(0, 1, 3e-3, 1e-4) == pytest.approx(3e-3)
    assert math.isnan(q.aqn_sigma(0, 10, 0.0, 1e-4))


FAKE = 1 << 20  # a 16-byte-aligned address that is never dereferenced
P = ctypes.c_void_p


def _quant(**kw):
    a = dict(w=FAKE, n=4, k=32, ldw=32, packed=FAKE, scales=FAKE, ts=FAKE, ts_in=None, flags=0,
             ws=FAKE, ws_bytes=1 << 16, stream=None)
    a.update(kw)
    return q.lib().qerl_nvfp4_quantize(P(a["w"]), a["n"], a["k"], a["ldw"], P(a["packed"]),
                                       P(a["scales"]), P(a["ts"]), P(a["ts_in"]), a["flags"],
                                       P(a["ws"]), a["ws_bytes"], P(a["stream"]))


@pytest.mark.parametrize("kw,status", [
    (dict(w=None), 1), (dict(packed=None), 1), (dict(scales=None), 1), (dict(ts=None), 1),
    (dict(n=0), 2), (dict(k=24, ldw=24), 2), (dict(k=0, ldw=0), 2), (dict(ldw=16), 2),
    (dict(w=FAKE + 2), 3), (dict(packed=FAKE + 8), 3), (dict(ldw=36), 3),
    (dict(flags=2), 4), (dict(ws=None), 5), (dict(ws_bytes=16), 5), (dict(ws=FAKE + 4), 3),
])
def test_quantize_argument_errors(kw, status):
    assert _quant(**kw) == status
    assert q.lib().qerl_last_error()


def _gemm(**kw):
    a = dict(x=FAKE, m=2, k=64, ldx=64, packed=FAKE, scales=FAKE, ts=FAKE, n=32, A=FAKE, B=FAKE,
             r=4, lam=2.0, y=FAKE, ldy=32, ws=FAKE, ws_bytes=1 << 16, stream=None)
    a.update(kw)
    return q.lib().qerl_w4a16_lora_gemm(P(a["x"]), a["m"], a["k"], a["ldx"], P(a["packed"]),
                                        P(a["scales"]), P(a["ts"]), a["n"], P(a["A"]), P(a["B"]),
                                        a["r"], a["lam"], P(a["y"]), a["ldy"], P(a["ws"]),
                                        a["ws_bytes"], P(a["stream"]))


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(y=None), 1), (dict(ts=None), 1), (dict(A=None), 1),
    (dict(r=-1), 4), (dict(r=129), 4), (dict(lam=float("nan")), 4), (dict(lam=float("inf")), 4),
    (dict(m=0), 2), (dict(n=0), 2), (dict(k=40, ldx=40), 2), (dict(ldx=48), 2), (dict(ldy=16), 2),
    (dict(x=FAKE + 2), 3), (dict(y=FAKE + 1), 3), (dict(A=FAKE + 8), 3), (dict(ldx=68), 3),
    (dict(ts=FAKE + 2), 3), (dict(ws=None), 5), (dict(ws_bytes=8), 5),
])
def test_gemm_argument_errors(kw, status):
    assert _gemm(**kw) == status


def test_gemm_without_lora_needs_no_lora_pointers_or_workspace_check():
    # r == 0: A/B may be NULL; still rejected here on a bad shape, before any launch
    assert _gemm(r=0, A=None, B=None, ws=None, ws_bytes=0, m=0) == 2


def _aqn(**kw):
    a = dict(x=FAKE, m=2, h=64, ldx=64, w=FAKE, eps=1e-6, sigma=1e-2, seed=1, step=0, layer=0,
             yf=FAKE, yb=None, ldy=64, wn=None, stream=None)
    a.update(kw)
    return q.lib().qerl_aqn_rmsnorm(P(a["x"]), a["m"], a["h"], a["ldx"], P(a["w"]), a["eps"],
                                    a["sigma"], a["seed"], a["step"], a["layer"], P(a["yf"]),
                                    P(a["yb"]), a["ldy"], P(a["wn"]), P(a["stream"]))


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(w=None), 1), (dict(yf=None, yb=None), 1),
    (dict(m=0), 2), (dict(h=0), 2), (dict(h=16385, ldx=16392, ldy=16392), 2), (dict(ldx=32), 2),
    (dict(x=FAKE + 1), 3), (dict(w=FAKE + 2), 3), (dict(wn=FAKE + 2), 3), (dict(yf=FAKE + 1), 3),
    (dict(eps=0.0), 4), (dict(eps=-1.0), 4), (dict(eps=float("inf")), 4),
    (dict(sigma=-1e-3), 4), (dict(sigma=float("nan")), 4),
])
def test_aqn_argument_errors(kw, status):
    assert _aqn(**kw) == status


def test_workspace_queries():
    assert q.nvfp4_quantize_workspace_size(27648, 5120) >= 4096
    assert q.w4a16_lora_gemm_workspace_size(64, 3584, 3584, 32) >= 64 * 32 * 4
    # decode sizes keep FP32 split-K partials: at least one m x n slice
    assert q.w4a16_lora_gemm_workspace_size(1, 3584, 3584, 0) >= 3584 * 4


def _multi(nseg=3, segs_kw=None, **kw):
    a = dict(x=FAKE, m=2, k=64, ldx=64, ws=FAKE, ws_bytes=1 << 24, stream=None, segs=True)
    a.update(kw)
    arr = (q.GemmSegment * max(nseg, 1))()
    for i in range(max(nseg, 1)):
        s = dict(packed=FAKE, scales=FAKE, ts=FAKE, n=32 + 16 * i, A=FAKE, B=FAKE, r=4, lam=2.0, y=FAKE, ldy=64)
        s.update((segs_kw or {}).get(i, {}))
        arr[i] = q.GemmSegment(s["packed"], s["scales"], s["ts"], s["n"], s["A"], s["B"], s["r"], s["lam"],
                               s["y"], s["ldy"])
    return q.lib().qerl_w4a16_lora_gemm_multi(P(a["x"]), a["m"], a["k"], a["ldx"], arr if a["segs"] else None,
                                              nseg, P(a["ws"]), a["ws_bytes"], P(a["stream"]))


@pytest.mark.parametrize("nseg,segs_kw,kw,status", [
    (3, None, dict(segs=False), 1), (0, None, {}, 4), (5, None, {}, 4), (3, None, dict(x=None), 1),
    (3, {1: dict(y=None)}, {}, 1), (3, {2: dict(r=200)}, {}, 4), (3, {0: dict(n=0)}, {}, 2),
    (3, {1: dict(A=FAKE + 4)}, {}, 3), (3, {2: dict(ldy=8)}, {}, 2), (2, None, dict(k=40, ldx=40), 2),
    (3, None, dict(ws=None), 5), (3, None, dict(ws_bytes=64), 5), (3, None, dict(ws=FAKE + 8), 3),
])
def test_gemm_multi_argument_errors(nseg, segs_kw, kw, status):
    assert _multi(nseg, segs_kw, **kw) == status
    assert q.lib().qerl_last_error()


def test_gemm_multi_workspace_query():
    shapes = [(3584, 32), (512, 32), (512, 32)]
    # decode sizes: one region per segment
    for m in (1, 8, 64, 128, 256):
        total = q.w4a16_lora_gemm_multi_workspace_size(m, 3584, shapes)
        assert total >= 3 * 64 * 1024
    # large m (above 256) runs the segments in turn over one region: the largest single need
    big = q.w4a16_lora_gemm_multi_workspace_size(257, 3584, shapes)
    assert big == max(q.w4a16_lora_gemm_workspace_size(257, n, 3584, r) for n, r in shapes)
    assert q.lib().qerl_w4a16_lora_gemm_multi_workspace_size(1, 3584, None, 3) == 0


def _norm_multi(nseg=2, segs_kw=None, **kw):
    a = dict(x=FAKE, m=2, k=64, ldx=64, nw=FAKE, eps=1e-6, ws=FAKE, ws_bytes=1 << 24, stream=None, segs=True)
    a.update(kw)
    arr = (q.GemmSegment * max(nseg, 1))()
    for i in range(max(nseg, 1)):
        s = dict(packed=FAKE, scales=FAKE, ts=FAKE, n=32 + 16 * i, A=FAKE, B=FAKE, r=4, lam=2.0, y=FAKE, ldy=64)
        s.update((segs_kw or {}).get(i, {}))
        arr[i] = q.GemmSegment(s["packed"], s["scales"], s["ts"], s["n"], s["A"], s["B"], s["r"], s["lam"],
                               s["y"], s["ldy"])
    return q.lib().qerl_rmsnorm_w4a16_lora_gemm_multi(P(a["x"]), a["m"], a["k"], a["ldx"], P(a["nw"]), a["eps"],
                                                      arr if a["segs"] else None, nseg, P(a["ws"]), a["ws_bytes"],
                                                      P(a["stream"]))


@pytest.mark.parametrize("nseg,segs_kw,kw,status", [
    (2, None, dict(segs=False), 1), (2, None, dict(nw=None), 1), (0, None, {}, 4), (5, None, {}, 4),
    (2, None, dict(eps=0.0), 4), (2, None, dict(eps=float("nan")), 4), (2, None, dict(nw=FAKE + 4), 3),
    (2, None, dict(k=16400, ldx=16400), 2), (2, None, dict(x=None), 1), (2, {1: dict(r=-1)}, {}, 4),
    (2, {0: dict(n=0)}, {}, 2), (2, None, dict(ws=None), 5), (2, None, dict(ws_bytes=64), 5),
    (2, None, dict(ws=FAKE + 8), 3),
])
def test_norm_gemm_multi_argument_errors(nseg, segs_kw, kw, status):
    assert _norm_multi(nseg, segs_kw, **kw) == status
    assert q.lib().qerl_last_error()


def test_norm_gemm_multi_workspace_query():
    shapes = [(3584, 32), (512, 32), (512, 0)]
    # fused (m <= 16, k % 32 == 0): the decode regions plus the producers' sums of squares
    for m in (1, 8, 16):
        fused = q.rmsnorm_w4a16_lora_gemm_multi_workspace_size(m, 3584, shapes)
        assert fused >= q.w4a16_lora_gemm_multi_workspace_size(m, 3584, shapes)
    # otherwise the GEMM's workspace, then room for the normed rows
    for m, k in ((24, 3584), (100, 3584), (4, 3600)):
        plain = q.w4a16_lora_gemm_multi_workspace_size(m, k, shapes)
        assert q.rmsnorm_w4a16_lora_gemm_multi_workspace_size(m, k, shapes) >= plain + m * k * 2
    assert q.lib().qerl_rmsnorm_w4a16_lora_gemm_multi_workspace_size(1, 3584, None, 2) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(w=None), 1), (dict(out=None), 1), (dict(h=0), 2), (dict(h=16385), 2), (dict(w=FAKE + 2), 3),
    (dict(out=FAKE + 1), 3), (dict(sigma=-1.0), 4), (dict(sigma=float("inf")), 4),
])
def test_aqn_noisy_weight_argument_errors(kw, status):
    a = dict(w=FAKE, h=64, sigma=1e-2, seed=1, step=0, layer=0, out=FAKE, stream=None)
    a.update(kw)
    assert q.lib().qerl_aqn_noisy_weight(P(a["w"]), a["h"], a["sigma"], a["seed"], a["step"], a["layer"],
                                         P(a["out"]), P(a["stream"])) == status


@pytest.mark.parametrize("kw,status", [
    (dict(w=None), 1), (dict(packed=None), 1), (dict(scales=None), 1), (dict(n=0), 2), (dict(k=48, ldw=48), 2),
    (dict(k=16, ldw=16), 2), (dict(ldw=32), 2), (dict(w=FAKE + 2), 3), (dict(packed=FAKE + 8), 3),
    (dict(ldw=68), 3),
])
def test_mxfp4_argument_errors(kw, status):
    a = dict(w=FAKE, n=4, k=64, ldw=64, packed=FAKE, scales=FAKE, stream=None)
    a.update(kw)
    assert q.lib().qerl_mxfp4_quantize(P(a["w"]), a["n"], a["k"], a["ldw"], P(a["packed"]), P(a["scales"]),
                                       P(a["stream"])) == status
    assert q.lib().qerl_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(w=None), 1), (dict(n=0), 2), (dict(k=24, ldw=24), 2), (dict(flags=4), 4), (dict(ws=None), 5),
])
def test_quantize_stochastic_argument_errors(kw, status):
    a = dict(w=FAKE, n=4, k=64, ldw=64, packed=FAKE, scales=FAKE, ts=FAKE, flags=0, seed=1, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    assert q.lib().qerl_nvfp4_quantize_stochastic(P(a["w"]), a["n"], a["k"], a["ldw"], P(a["packed"]),
                                                  P(a["scales"]), P(a["ts"]), None, a["flags"], a["seed"],
                                                  P(a["ws"]), a["wsb"], None) == status
    assert b"nvfp4_quantize_stochastic" in q.lib().qerl_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(dy=None), 1), (dict(x=None), 1), (dict(A=None), 1), (dict(r=200), 4), (dict(lam=float("inf")), 4),
    (dict(m=0), 2), (dict(k=40, ldx=40, lddx=40), 2), (dict(ldy=16), 2), (dict(lddx=8), 2),
    (dict(dy=FAKE + 2), 3), (dict(x=FAKE + 4), 3), (dict(ldx=68), 3), (dict(dx=FAKE + 1), 3),
    (dict(ws=None), 5), (dict(wsb=16), 5), (dict(ws=FAKE + 8), 3),
])
def test_backward_argument_errors(kw, status):
    a = dict(dy=FAKE, m=4, n=32, ldy=32, x=FAKE, k=64, ldx=64, packed=FAKE, scales=FAKE, ts=FAKE, A=FAKE, B=FAKE,
             r=8, lam=2.0, dx=FAKE, lddx=64, da=FAKE, db=FAKE, ws=FAKE, wsb=1 << 24)
    a.update(kw)
    assert q.lib().qerl_w4a16_lora_backward(P(a["dy"]), a["m"], a["n"], a["ldy"], P(a["x"]), a["k"], a["ldx"],
                                            P(a["packed"]), P(a["scales"]), P(a["ts"]), P(a["A"]), P(a["B"]),
                                            a["r"], a["lam"], P(a["dx"]), a["lddx"], P(a["da"]), P(a["db"]),
                                            P(a["ws"]), a["wsb"], None) == status
    assert q.lib().qerl_last_error()


def test_backward_workspace_query():
    assert q.w4a16_lora_backward_workspace_size(2048, 5120, 5120, 32) >= 2 * 2048 * 32 * 4
    assert q.w4a16_lora_backward_workspace_size(0, 5120, 5120, 32) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(packed=None), 1), (dict(scales=None), 1), (dict(ts=None), 1), (dict(out=None), 1), (dict(n=0), 2),
    (dict(k=24, ldo=24), 2), (dict(k=0, ldo=16), 2), (dict(ldo=32), 2), (dict(packed=FAKE + 4), 3),
    (dict(out=FAKE + 8), 3), (dict(ldo=68), 3), (dict(ts=FAKE + 2), 3),
])
def test_dequantize_argument_errors(kw, status):
    a = dict(packed=FAKE, scales=FAKE, ts=FAKE, n=4, k=64, out=FAKE, ldo=64, stream=None)
    a.update(kw)
    assert q.lib().qerl_nvfp4_dequantize(P(a["packed"]), P(a["scales"]), P(a["ts"]), a["n"], a["k"], P(a["out"]),
                                         a["ldo"], P(a["stream"])) == status
    assert q.lib().qerl_last_error()


def test_last_hip_error_is_the_error_text():
    L = q.lib()
    assert L.qerl_w4a16_lora_gemm(None, 1, 16, 16, None, None, None, 1, None, None, 0, 0.0, None, 1, None, 0,
                                  None) == 1
    assert L.qerl_last_error() and L.qerl_last_hip_error() == L.qerl_last_error()


def test_noalloc_gemm_rejects_sizes_above_the_scratch():
    """Host-side checks of qerl_w4a16_lora_gemm_noalloc: nothing is enqueued
    (the pointers are never dereferenced)."""
    L = q.lib()
    m, n, k, r = 128, 27648, 5120, 32
    assert L.qerl_w4a16_lora_gemm_workspace_size(m, n, k, r) > q.NOALLOC_SCRATCH_BYTES
    st = L.qerl_w4a16_lora_gemm_noalloc(P(FAKE), m, k, k, P(FAKE), P(FAKE), P(FAKE), n, P(FAKE), P(FAKE), r, 2.0,
                                        P(FAKE), n, None)
    assert st == 5  # QERL_ERR_WORKSPACE
    assert b"scratch" in L.qerl_last_hip_error()
    # argument checks come first, as in the workspace call
    st = L.qerl_w4a16_lora_gemm_noalloc(None, 1, 16, 16, P(FAKE), P(FAKE), P(FAKE), 1, None, None, 0, 0.0,
                                        P(FAKE), 1, None)
    assert st == 1  # QERL_ERR_NULL
