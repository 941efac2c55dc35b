"""The C ABI layer (exact_attention_flash_amd/csrc/flash_attn.cpp) built for the host
alone under AddressSanitizer and UndefinedBehaviorSanitizer, with the device
launchers stubbed (tests/host_sanitize/abi_fuzz.cpp), and driven through every
entry point: known good and bad arguments, then random ones at the integer limits.
Catches signed overflow in the size and overlap arithmetic, out-of-bounds reads of
the stride arrays and the like; no GPU is involved.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_flash_amd", "csrc")
ROCM_INC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INC), reason="g++ or ROCm headers missing")
def test_abi_layer_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "abi_fuzz")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INC}",
               f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", os.path.join(CSRC, "flash_attn.cpp"),
               os.path.join(ROOT, "tests", "host_sanitize", "abi_fuzz.cpp"), "-o", exe]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        run = subprocess.run([exe, "300000"], capture_output=True, text=True, env=env, timeout=300)
        assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
        assert "0 failed checks" in run.stdout
