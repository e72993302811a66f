"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds every library source with the sanitizers on the host side only (hipcc's
``-Xarch_host``; the device code is compiled as usual and never runs here), links
``capi_host_check.cpp`` against those objects with ROCm's clang, and runs it: every
entry point is called with arguments its host checks must reject before anything is
enqueued.  A sanitizer report, or a status code other than the expected one, fails
the test.
"""

import os
import shutil
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "packed_sequence_block_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain not found")
def test_host_argument_checks_under_asan_ubsan(tmp_path):
    objs = []
    for src in ("boundary.hip", "schedule.hip", "attn_fwd.hip", "attn_bwd.hip"):
        obj = str(tmp_path / (src + ".o"))
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-sanitize-recover=undefined",
                        "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj],
                       check=True, capture_output=True)
        objs.append(obj)
    exe = str(tmp_path / "capi_host_check")
    subprocess.run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-I", INCLUDE,
                    os.path.join(ROOT, "tests", "capi_host_check.cpp"), os.path.join(CSRC, "capi.cpp")] + objs +
                   ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                   check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "host checks ok" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
    shutil.rmtree(tmp_path, ignore_errors=True)
