"""The C ABI layer built with AddressSanitizer and UndefinedBehaviorSanitizer
on the host code and driven through every entry point (no GPU needed).

tests/native/abi_sanitized.cpp calls each function of include/mlstm.h,
slstm.h and mlstm_prof.h through its argument checks and, with host-only
stand-in launchers (tests/native/abi_stub_launchers.cpp), through its
workspace carving and dispatch. The sanitizers instrument only the host
code (each -fsanitize= follows -Xarch_host); the build compiles
csrc/mlstm_abi.cpp as it is, its one device array included.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "tests", "native", "abi_sanitized.cpp"),
           os.path.join(ROOT, "tests", "native", "abi_stub_launchers.cpp"),
           os.path.join(ROOT, "linear_recurrent_sequence_fwd_amd", "csrc", "mlstm_abi.cpp")]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_abi_layer_under_asan_and_ubsan(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_sanitized")
    cmd = [hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(ROOT, "include"), "-o", exe, *SOURCES]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "all expectations held" in run.stdout
    assert "ERROR: AddressSanitizer" not in run.stderr
    assert "runtime error" not in run.stderr
