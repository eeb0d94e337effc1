"""The C ABI from C: tests/c_caller.c, compiled as C99 with gcc against
include/rlk.h and linked against librlk.so, runs and gets the documented
answers (CPU only: it calls no entry point that launches)."""
import os
import shutil
import subprocess

import pytest

import invariant_logprob_amd as ilp
from invariant_logprob_amd import build as rlk_build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_caller(tmp_path):
    if not os.path.exists(ilp.library_path()):
        rlk_build.build()
    libdir = os.path.dirname(ilp.library_path())
    exe = str(tmp_path / "c_caller")
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror=implicit-function-declaration",
           "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROCM, 'include')}",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(HERE, "c_caller.c"),
           f"-L{libdir}", "-l:librlk.so", f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c caller ok" in r.stdout, r.stdout + r.stderr
