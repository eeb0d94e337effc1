"""No atomic instruction anywhere in the library's gfx950 code: every
reduction must have a fixed order (page "[WS1 Test] #154 dtype pin + ...",
section "Workstream 3 - #153", scope item 2: no atomicAdd).  Scans the AMD
assembly of this repository's own sources (CPU only; hipcc cross-compiles)."""
import os
import re
import subprocess

import pytest

from invariant_logprob_amd import build as rlk_build

CSRC = os.path.join(rlk_build.PKG, "csrc")


@pytest.mark.parametrize("src", rlk_build.SOURCES)
def test_device_code_has_no_atomics(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [rlk_build.HIPCC, *rlk_build.COMMON, "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    hits = [l.strip() for l in asm.splitlines()
            if re.match(r"\s*(buffer|global|flat|ds|scratch)_atomic", l)]
    assert not hits, hits[:5]
    # the kernels exist in this object (the scan looked at real code); the
    # host-side sources hold none (noalloc.hip only a device array)
    if src not in ("rlk_api.hip", "noalloc.hip"):
        assert ".amdhsa_kernel" in asm
    if src == "noalloc.hip":
        assert "scratch" in asm
