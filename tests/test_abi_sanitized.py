"""The C ABI's host-side argument validation (csrc/rlk_api.hip) built for the
host alone under AddressSanitizer and UndefinedBehaviorSanitizer, linked
against stand-in launchers (tests/abi_sanitized_driver.cpp) and run on the
CPU: every documented status, a launch reached exactly on valid arguments,
and no memory error or signed overflow in the size arithmetic at the limits.
No device code is built or run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
INC = [f"-I{os.path.join(ROOT, 'include')}",
       f"-I{os.path.join(ROOT, 'invariant_logprob_amd', 'csrc')}"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="needs the ROCm compilers")
def test_validation_under_host_sanitizers(tmp_path):
    api = str(tmp_path / "api.o")
    drv = str(tmp_path / "driver.o")
    exe = str(tmp_path / "abi_sanitized")
    # host pass only: no device code, and each sanitizer flag scoped to the host
    steps = [
        [HIPCC, "--cuda-host-only", "-x", "hip", "-std=c++17", "-O1", "-g",
         "-fno-omit-frame-pointer",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=all", *INC,
         "-c", os.path.join(ROOT, "invariant_logprob_amd", "csrc", "rlk_api.hip"), "-o", api],
        [CLANGXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
         f"-I{os.path.join(ROCM, 'include')}", *INC, "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-c", os.path.join(HERE, "abi_sanitized_driver.cpp"),
         "-o", drv],
        [CLANGXX, "-fsanitize=address,undefined", api, drv, "-o", exe],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, " ".join(cmd) + "\n" + r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "sanitized validation ok" in r.stdout, r.stdout + r.stderr[-3000:]
