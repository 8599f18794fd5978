"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU lane).

tests/abi_sanitize_driver.cpp is linked with the library's sources, built with the sanitizers on
the host side only (each -fsanitize= after -Xarch_host; the device code is built as usual), and
run: it calls every entry point with sizes at and past the documented bounds and with null,
misaligned and fake pointers, and checks the statuses.  Any out-of-bounds access or signed
overflow in the validation and workspace arithmetic aborts the run.  No call reaches a kernel
launch: without a GPU, arguments that validate stop at the device query (LMH_ERR_HIP)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lm_head_log_lmhead_amd", "csrc")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_host_validation_under_asan_and_ubsan(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_sanitize_driver")
    san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                 "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", flag]
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-g", "-std=c++17", *san,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
           f"-I{ROOT}/include", f"-I{CSRC}",
           *[os.path.join(CSRC, f) for f in ("api.hip", "fwd.hip", "bwd.hip")],
           "-x", "hip", os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    import torch
    have_gpu = torch.cuda.device_count() > 0
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, "1" if have_gpu else "0"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "abi sanitize driver ok" in r.stdout
