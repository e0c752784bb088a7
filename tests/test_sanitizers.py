"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU (no GPU).

- The forward and backward oracles (oracle/*.c) are compiled with gcc and
  both sanitizers and driven over small inputs that reach every branch of
  their token loops (tests/sanitize/oracle_driver.c).
- The library (argument validation, workspace sizing, the status and
  error-string paths of every entry point) is built with the same sanitizers
  on its host code only (the gfx950 device code is built as usual) and driven
  through include/kda.h with requests that are rejected before any GPU work
  (tests/sanitize/abi_driver.c).

Any sanitizer report aborts the driver, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "gated_delta_rule_33_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LIB_SOURCES = ["kda_api.cpp", "kda_prep.hip", "kda_intra.hip", "kda_fused.hip", "kda_recur.hip", "kda_layer.hip",
               "kda_cp.hip", "kda_bwd.hip"]
# Host-side sanitizer flags, each behind -Xarch_host so no device code is built with them.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-DREAL=double", "-o", exe, os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "kda_oracle.c"), os.path.join(ROOT, "oracle", "kda_oracle_bwd.c"),
          "-lm", "-lpthread"])
    r = _run([exe], env=ENV, timeout=300)
    assert r.stdout.strip().endswith("ok")


def test_abi_validation_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    objs = []
    procs = []
    for src in LIB_SOURCES:
        obj = str(tmp_path / (src + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen(
            [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC, *HOST_SAN, "-c", os.path.join(CSRC, src),
             "-o", obj], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p, src in zip(procs, LIB_SOURCES):
        out, err = p.communicate()
        assert p.returncode == 0, f"{src}\n{err}"
    lib = str(tmp_path / "libkda_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, "-o", lib, *objs])
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, "--offload-host-only", "-O1", "-g", "-x", "c", *HOST_SAN, "-I", os.path.join(ROOT, "include"),
          "-o", exe, os.path.join(HERE, "abi_driver.c"), "-x", "none", lib, f"-Wl,-rpath,{tmp_path}", "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert r.stdout.strip().endswith("ok")
