"""The C ABI's host code (argument validation, workspace layouts, error
text) built with AddressSanitizer and UndefinedBehaviorSanitizer on the
host side and run over every validation path (tests/sanitize/
host_checks.cpp). No GPU: every call there is refused before a launch or
only sizes a workspace."""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "verified_sparse_kv_amd", "csrc")
SOURCES = ["vkv_api", "vkv_compress", "vkv_decode", "vkv_dense", "vkv_sketch2",
           "vkv_maint"]
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/bin/amdclang++"


@pytest.mark.timeout(900)
@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="ROCm compilers not installed")
def test_host_code_under_asan_and_ubsan():
    # each -fsanitize= applies to the host compilation only (-Xarch_host)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    common = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory() as td:
        objs = []
        for s in SOURCES:
            o = os.path.join(td, s + ".o")
            cmd = [HIPCC, "--offload-arch=gfx950", "-Xclang", "-target-feature",
                   "-Xclang", "-packed-fp32-ops"] + common + san + \
                  ["-c", os.path.join(CSRC, s + ".hip"), "-o", o]
            subprocess.run(cmd, check=True, capture_output=True)
            objs.append(o)
        drv = os.path.join(td, "host_checks.o")
        subprocess.run([CLANG] + common + ["-fsanitize=address", "-fsanitize=undefined",
                       "-c", os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"),
                       "-o", drv], check=True, capture_output=True)
        exe = os.path.join(td, "host_checks")
        subprocess.run([HIPCC, "--offload-arch=gfx950"] + san + objs + [drv, "-o", exe],
                       check=True, capture_output=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
                   HIP_VISIBLE_DEVICES="")
        res = subprocess.run([exe], env=env, capture_output=True, text=True,
                             timeout=300)
        out = res.stdout + res.stderr
        assert res.returncode == 0, out[-4000:]
        assert "host checks: 0 failures" in out
        assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
