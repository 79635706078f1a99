"""Host argument validation under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/abi_validate.c calls every entry point with arguments that
must be rejected (or, for size queries, answered) on the host, against a
build whose host code (dg_api.hip) is instrumented; the kernels are the
regular build's.  No GPU is touched: every call returns before any HIP
call.  A sanitizer report or a wrong status fails the test."""
import os
import shutil
import subprocess

import pytest

from discrete_text_diffusion_step_amd import build as dgbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not (os.path.exists(CLANG) and shutil.which(dgbuild.HIPCC) or os.path.exists(dgbuild.HIPCC)),
                    reason="needs the ROCm clang and hipcc")
def test_host_validation_under_asan_ubsan(tmp_path):
    lib = dgbuild.build_host_sanitized(str(tmp_path))
    exe = str(tmp_path / "abi_validate")
    src = os.path.join(ROOT, "tests", "sanitize", "abi_validate.c")
    cmd = [CLANG, "-std=c11", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"), src, lib,
           f"-Wl,-rpath,{tmp_path}", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " 0 failed" in r.stdout, r.stdout
