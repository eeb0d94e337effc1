"""Build librlk.so (the HIP library behind include/rlk.h) for gfx950.

    python -m invariant_logprob_amd.build

Each HIP source is compiled with hipcc for gfx950 only, in parallel, into
``_build/`` and linked in-tree as ``invariant_logprob_amd/librlk.so``.  Packed
fp32 instructions are disabled for all device code.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librlk.so")
SOURCES = ["rlk_api.hip", "logits_rows.hip", "linear_tiles.hip", "linear_grads.hip", "token_losses.hip",
           "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def git_rev():
    try:
        rev = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"],
                             capture_output=True, text=True, timeout=10).stdout.strip()
        dirty = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--", "invariant_logprob_amd/csrc",
                                "include"], capture_output=True, text=True, timeout=10).stdout.strip()
        return (rev or "unknown") + ("+dirty" if dirty else "")
    except Exception:
        return "unknown"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that notice is harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    defs = [f'-DRLK_GIT_REV="{git_rev()}"']
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *COMMON, *defs, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        for err in ex.map(_run, cmds):
            if verbose and err:
                print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


YARDSTICK_SRC = os.path.join(ROOT, "yardstick", "yardstick.hip")
YARDSTICK_LIB = os.path.join(ROOT, "yardstick", "libyardstick.so")


def build_yardstick():
    """The benchmark's measurement kernels (attainable read and matrix rates,
    shader clock): a library of their own, never linked into librlk.so."""
    tmp = YARDSTICK_LIB + ".tmp"
    _run([HIPCC, *COMMON, "-shared", YARDSTICK_SRC, "-o", tmp])
    os.replace(tmp, YARDSTICK_LIB)
    return YARDSTICK_LIB


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_yardstick())
