"""The C-ABI library loads, exports what include/rlk.h declares, and rejects
bad arguments before any launch (CPU only: validation never touches the GPU)."""
import ctypes
import os
import re

import pytest

import invariant_logprob_amd as ilp
from invariant_logprob_amd import build as rlk_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rlk.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ilp.library_path()):
        rlk_build.build()
    return ilp.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rlk_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("rlk_logp_selected", "rlk_linear_logp", "rlk_logp_backward",
              "rlk_linear_logp_workspace_size", "rlk_status_string", "rlk_build_info"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_build_info_and_status_strings(lib):
    info = ilp.build_info()
    assert "gfx950" in info and "rlk" in info
    assert lib.rlk_status_string(0) == b"RLK_OK"
    assert lib.rlk_status_string(2) == b"RLK_ERR_UNSUPPORTED"
    assert lib.rlk_status_string(99) == b"unknown"


# Fake device addresses: validation rejects before any launch, so these are
# never dereferenced.  A16 is 16-byte aligned, A2 is not.
A16 = ctypes.c_void_p(0x10000)
A2 = ctypes.c_void_p(0x10002)
NUL = None


def test_logp_selected_validation(lib):
    f = lib.rlk_logp_selected
    assert f(A16, 1024, A16, NUL, 0, 1024, A16, NUL, NUL) == OK          # N == 0: no-op
    assert f(A16, 1024, A16, NUL, -1, 1024, A16, NUL, NUL) == INVALID
    assert f(A16, 1024, A16, NUL, 4, 0, A16, NUL, NUL) == INVALID        # V < 1
    assert f(NUL, 1024, A16, NUL, 4, 1024, A16, NUL, NUL) == INVALID     # no logits
    assert f(A16, 1024, NUL, NUL, 4, 1024, A16, NUL, NUL) == INVALID     # no targets
    assert f(A16, 1024, A16, NUL, 4, 1024, NUL, NUL, NUL) == INVALID     # no logp
    assert f(A16, 1000, A16, NUL, 4, 1024, A16, NUL, NUL) == INVALID     # ld < V
    assert f(A16, 1028, A16, NUL, 4, 1024, A16, NUL, NUL) == UNSUPPORTED  # ld % 8
    assert f(A2, 1024, A16, NUL, 4, 1024, A16, NUL, NUL) == UNSUPPORTED   # misaligned
    assert f(A16, 1 << 29, A16, NUL, 4, 1 << 29, A16, NUL, NUL) == UNSUPPORTED  # V too large


def test_linear_logp_validation(lib):
    f = lib.rlk_linear_logp
    ws = lib.rlk_linear_logp_workspace_size(300, 1000, 64)
    assert ws >= 4 * 300 * 8 + 300 * 4
    args = lambda **k: [k.get("h", A16), k.get("ldh", 64), k.get("w", A16), k.get("ldw", 64),
                        A16, NUL, k.get("n", 300), k.get("v", 1000), k.get("H", 64), A16, NUL,
                        k.get("ws", A16), k.get("wsb", ws), NUL]
    assert f(*args(n=0)) == OK
    assert f(*args(H=0)) == INVALID
    assert f(*args(ldh=56)) == INVALID                     # ld_h < H
    assert f(*args(wsb=ws - 1)) == INVALID                 # workspace too small
    assert f(*args(ws=NUL)) == INVALID
    assert f(*args(H=60, ldh=64, ldw=64)) == UNSUPPORTED   # H % 8
    assert f(*args(ldw=68)) == UNSUPPORTED                 # ld_w % 8
    assert f(*args(w=A2)) == UNSUPPORTED
    assert f(*args(ws=A2)) == UNSUPPORTED


def test_backward_validation(lib):
    f = lib.rlk_logp_backward
    base = dict(lg=A16, ld=1024, h=NUL, ldh=0, w=NUL, ldw=0, H=0, t=A16, m=NUL, lse=A16, g=A16,
                n=4, v=1024, out=A16, ldg=1024)
    call = lambda **k: f(*[{**base, **k}[x] for x in ("lg", "ld", "h", "ldh", "w", "ldw", "H", "t",
                                                      "m", "lse", "g", "n", "v", "out", "ldg")], NUL)
    assert call(n=0) == OK
    assert call(lse=NUL) == INVALID
    assert call(g=NUL) == INVALID
    assert call(ldg=1000) == INVALID
    assert call(ldg=1026) == UNSUPPORTED
    assert call(out=ctypes.c_void_p(0x10008)) == UNSUPPORTED
    # fused mode (logits NULL) needs hidden and weight
    assert call(lg=NUL) == INVALID
    assert call(lg=NUL, h=A16, ldh=64, w=A16, ldw=64, H=0) == INVALID
    assert call(lg=NUL, h=A16, ldh=64, w=A2, ldw=64, H=64) == UNSUPPORTED
    # logits mode reads bf16 and writes fp32: an output span that overlaps the
    # logits' is refused (4 rows of 1024 bf16 span 8 KB from 0x10000)
    assert call(out=A16) == INVALID
    assert call(out=ctypes.c_void_p(0x10000 + 8 * 1024 - 16)) == INVALID   # ends of the spans
    assert call(out=ctypes.c_void_p(0x10000 - 4 * (3 * 1024 + 1024) + 16)) == INVALID


def test_dense_log_softmax_refuses_overlap(lib):
    g = lib.rlk_log_softmax
    assert g(A16, 1024, NUL, A16, 4, 1024, A16, 1024, NUL) == INVALID      # same base
    assert g(A16, 1024, NUL, A16, 4, 1024, ctypes.c_void_p(0x10000 + 8 * 1024 - 16), 1024,
             NUL) == INVALID


def test_linear_logp_with_logits_validation(lib):
    f = lib.rlk_linear_logp_with_logits
    ws = lib.rlk_linear_logp_workspace_size(300, 1000, 64)
    args = lambda **k: [A16, 64, A16, 64, A16, NUL, k.get("n", 300), k.get("v", 1000), 64, A16,
                        NUL, k.get("z", A16), k.get("ldz", 1000), A16, k.get("wsb", ws), NUL]
    assert f(*args(n=0)) == OK
    assert f(*args(z=NUL)) == INVALID                     # the logits output is required
    assert f(*args(ldz=996)) == INVALID                   # ld_z < V
    assert f(*args(ldz=1002)) == UNSUPPORTED              # ld_z % 4
    assert f(*args(z=ctypes.c_void_p(0x10008))) == UNSUPPORTED   # misaligned
    assert f(*args(wsb=ws - 1)) == INVALID


def test_backward_f32_validation(lib):
    f = lib.rlk_logp_backward_f32
    base = dict(z=A16, ld=1024, t=A16, m=NUL, lse=A16, g=A16, n=4, v=1000, out=A16, ldg=1024)
    call = lambda **k: f(*[{**base, **k}[x] for x in ("z", "ld", "t", "m", "lse", "g", "n", "v",
                                                      "out", "ldg")], NUL)
    assert call(n=0) == OK
    assert call(z=NUL) == INVALID
    assert call(out=NUL) == INVALID
    assert call(lse=NUL) == INVALID
    assert call(g=NUL) == INVALID
    assert call(t=NUL) == INVALID
    assert call(ld=996) == INVALID                        # ld < V
    assert call(ld=1026, ldg=1026) == UNSUPPORTED         # ld % 4
    assert call(z=ctypes.c_void_p(0x10008)) == UNSUPPORTED
    # in place is the same buffer with the same stride; any other overlap is refused
    assert call(out=A16, ldg=1028) == INVALID
    assert call(out=ctypes.c_void_p(0x10000 + 16 * 4)) == INVALID
    assert call(out=ctypes.c_void_p(0x10000 + 3 * 1024 * 4)) == INVALID   # the last input row
    assert call(out=ctypes.c_void_p(0x10000 - 3 * 1024 * 4)) == INVALID   # ends in the first one


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(2, 8, dtype=torch.bfloat16)
    t = torch.zeros(2, dtype=torch.int64)
    with pytest.raises(ValueError):
        ilp.logp_selected(x, t)


def test_entropy_and_log_softmax_validation(lib):
    f = lib.rlk_logp_entropy
    assert f(A16, 1024, A16, NUL, 0, 1024, A16, NUL, A16, NUL) == OK
    assert f(A16, 1024, A16, NUL, 4, 1024, A16, NUL, NUL, NUL) == INVALID   # no entropy
    assert f(A16, 1024, NUL, NUL, 4, 1024, A16, NUL, A16, NUL) == INVALID   # no targets
    assert f(A16, 1028, A16, NUL, 4, 1024, A16, NUL, A16, NUL) == UNSUPPORTED
    g = lib.rlk_log_softmax
    assert g(A16, 1024, NUL, A16, 0, 1024, A16, 1024, NUL) == OK
    assert g(A16, 1024, NUL, NUL, 4, 1024, A16, 1024, NUL) == INVALID       # no lse
    assert g(A16, 1024, NUL, A16, 4, 1024, A16, 1000, NUL) == INVALID       # ld_out < V
    assert g(A16, 1024, NUL, A16, 4, 1024, A16, 1026, NUL) == UNSUPPORTED   # ld_out % 4
    assert g(A2, 1024, NUL, A16, 4, 1024, A16, 1024, NUL) == UNSUPPORTED


def test_token_losses_validation(lib):
    import ctypes as C
    f = lib.rlk_token_losses
    args = lambda **k: [k.get("lp", A16), k.get("old", A16), k.get("ref", NUL), k.get("adv", A16), NUL,
                        k.get("n", 10), C.c_float(k.get("lo", 0.2)), C.c_float(k.get("hi", 0.2)),
                        C.c_float(k.get("beta", 0.0)), k.get("r", A16), k.get("l", NUL), NUL, NUL, NUL]
    assert f(*args(n=0)) == OK
    assert f(*args(n=-1)) == INVALID
    assert f(*args(lp=NUL)) == INVALID
    assert f(*args(adv=NUL)) == INVALID
    assert f(*args(r=NUL)) == INVALID          # no output at all
    assert f(*args(lo=1.0)) == INVALID
    assert f(*args(beta=-0.1)) == INVALID


def test_linear_param_grads_validation(lib):
    f = lib.rlk_linear_logp_param_grads
    n, v, h = 300, 1000, 64
    ws = lib.rlk_linear_logp_param_grads_workspace_size(n, v, h)
    # one vocabulary chunk of D as two bf16 arrays (D_hi, D_lo), each [N, C],
    # C = V rounded up to 256 here, then a bf16 [N, H] copy of hidden with the
    # inactive rows zeroed
    c = 1024
    assert ws == 2 * ((n * c * 2 + 255) // 256 * 256) + (n * h * 2 + 255) // 256 * 256
    assert lib.rlk_linear_logp_param_grads_workspace_size(n, 200000, h) < \
        lib.rlk_linear_logp_param_grads_workspace_size(n, 20000, h) * 20   # chunked, not [N, V]

    def args(**k):
        return [k.get("h", A16), k.get("ldh", h), k.get("w", A16), k.get("ldw", h), k.get("t", A16),
                NUL, k.get("lse", A16), k.get("g", A16), k.get("n", n), k.get("v", v), k.get("H", h),
                k.get("gh", A16), k.get("ldgh", h), k.get("gw", A16), k.get("ldgw", h),
                k.get("ws", A16), k.get("wsb", ws), NUL]

    assert f(*args(gh=NUL, gw=NUL)) == INVALID            # nothing requested
    assert f(*args(n=-1)) == INVALID
    assert f(*args(v=0)) == INVALID
    assert f(*args(lse=NUL)) == INVALID
    assert f(*args(g=NUL)) == INVALID
    assert f(*args(t=NUL)) == INVALID
    assert f(*args(ws=NUL)) == INVALID
    assert f(*args(wsb=ws - 1)) == INVALID                 # workspace too small
    assert f(*args(ldgh=h - 4)) == INVALID
    assert f(*args(ldgw=h - 4)) == INVALID
    assert f(*args(ldgh=h + 2)) == UNSUPPORTED             # ld_gh % 4
    assert f(*args(gw=A2)) == UNSUPPORTED                  # misaligned output
    assert f(*args(H=60, ldh=64, ldw=64, ldgh=64, ldgw=64)) == UNSUPPORTED  # H % 8
    assert f(*args(n=1 << 22)) == UNSUPPORTED              # N beyond the transposed-operand range
    assert f(*args(ws=A2)) == UNSUPPORTED


def test_linear_param_grads_from_logits_validation(lib):
    f = lib.rlk_linear_logp_param_grads_from_logits
    n, v, h = 300, 1000, 64
    ws = lib.rlk_linear_logp_param_grads_workspace_size(n, v, h)

    def args(**k):
        return [k.get("z", A16), k.get("ldz", v), A16, h, A16, h, A16, NUL, A16, A16,
                k.get("n", n), v, h, k.get("gh", A16), h, k.get("gw", A16), h, A16,
                k.get("wsb", ws), NUL]

    assert f(*args(n=0, gw=NUL)) == OK                     # nothing to do, nothing launched
    assert f(*args(z=NUL)) == INVALID                      # the kept logits are required
    assert f(*args(ldz=v - 4)) == INVALID                  # ld_z < V
    assert f(*args(ldz=v + 2)) == UNSUPPORTED              # ld_z % 4
    assert f(*args(z=ctypes.c_void_p(0x10008))) == UNSUPPORTED   # misaligned
    assert f(*args(gh=NUL, gw=NUL)) == INVALID
    assert f(*args(wsb=ws - 1)) == INVALID


def test_linear_logp_noalloc_validation(lib):
    """The allocation-free fused forward checks its arguments like
    rlk_linear_logp and refuses, before touching any device, a problem whose
    chunk partials exceed its fixed 32 MiB array."""
    f = lib.rlk_linear_logp_noalloc

    def args(**k):
        return [k.get("h", A16), k.get("ldh", 4096), k.get("w", A16), k.get("ldw", 4096),
                k.get("t", A16), NUL, k.get("n", 8192), k.get("v", 128256), k.get("H", 4096),
                k.get("lp", A16), NUL, NUL]
    assert f(*args(n=0)) == OK                              # N == 0: no-op
    assert f(*args(t=NUL)) == INVALID
    assert f(*args(lp=NUL)) == INVALID
    assert f(*args(h=A2)) == UNSUPPORTED
    assert f(*args(ldh=4100)) == UNSUPPORTED
    # 501 chunk partials of 8 bytes + a target logit per row: 8363 rows fit in
    # 32 MiB at V = 128256, 8364 do not; at V = 151936 (594 chunks) 7055 fit
    assert lib.rlk_linear_logp_workspace_size(8363, 128256, 4096) <= 32 << 20
    assert lib.rlk_linear_logp_workspace_size(8364, 128256, 4096) > 32 << 20
    assert f(*args(n=8364)) == UNSUPPORTED
    assert lib.rlk_linear_logp_workspace_size(7055, 151936, 4096) <= 32 << 20
    assert f(*args(n=7056, v=151936)) == UNSUPPORTED
