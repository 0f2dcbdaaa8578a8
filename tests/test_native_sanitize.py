"""Sanitizer runs on the CPU (no GPU needed).

* The library's host code -- argument checks, size queries, launch plans --
  built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side
  only (``-Xarch_host`` before every -fsanitize flag; no kernel runs), driven by
  ``tests/native/host_checks.cpp``, which also checks every plan's workspace
  use against its size query for the decoder-layer shapes and a ragged sweep.
* The oracle (plain C) built the same way with gcc, and the oracle's own test
  files run against that build.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nvfp4_weight_only_quantize_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "api.cpp"),
                                                             os.path.join(ROOT, "tests", "native", "host_checks.cpp")]
    # device code is compiled as usual (and unsanitized): the host objects
    # need the code objects they register
    common = [HIPCC, "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"), *SAN_HOST]
    procs, objs = [], []
    for s in srcs:
        o = os.path.join(tmp_path, os.path.basename(s) + ".o")
        objs.append(o)
        procs.append((s, subprocess.Popen([*common, "-c", s, "-o", o], stdout=subprocess.PIPE,
                                          stderr=subprocess.STDOUT, text=True)))
    for s, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, f"host build of {os.path.basename(s)} failed:\n{out[-3000:]}"
    exe = os.path.join(tmp_path, "host_checks")
    _run([HIPCC, "--offload-arch=gfx950", *SAN_HOST, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env, timeout=600)
    assert "0 failed" in r.stdout, r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    lib = os.path.join(tmp_path, "libqerl_oracle_san.so")
    _run(["gcc", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-std=gnu11", "-shared", "-fPIC", "-pthread",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "qerl_oracle.c"), "-o", lib, "-lm"])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, QERL_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *tests],
         env=env, cwd=ROOT, timeout=900)
