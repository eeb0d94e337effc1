"""Shared helpers for the GPU parity and invariance tests."""
import numpy as np
import pytest
import torch

# Tolerances against the fp64 oracle (per element, r = oracle value)
def tol_logits(r):
    return 2e-5 + 1e-5 * np.abs(r)


TOL_FUSED = 2e-3
TOL_BWD = 1e-3


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def bits16(t):
    """Raw bf16 bits (numpy uint16) of a tensor, host copy."""
    return t.detach().contiguous().to("cpu").view(torch.int16).numpy().view(np.uint16)


def f32bits(t):
    return t.detach().contiguous().to("cpu").view(torch.int32)


def assert_close(got, ref, tol, what, active=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if active is not None:
        got = got[active]
        ref = ref[active]
    t = tol(ref) if callable(tol) else tol
    err = np.abs(got - ref)
    bad = ~(err <= t)
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at {tuple(idx)}: "
            f"got {got[tuple(idx)]!r} ref {ref[tuple(idx)]!r}; max err {np.nanmax(err):.3e}")
    return float(err.max()) if err.size else 0.0


def padded_bf16(n, v, ld, fill_rows):
    """[n, v] view of an [n, ld] bf16 buffer (ld % 8 == 0)."""
    buf = torch.empty((n, ld), dtype=torch.bfloat16, device=fill_rows.device)
    buf[:, v:] = float("nan")   # garbage beyond V must never be read
    buf[:, :v] = fill_rows
    return buf[:, :v]
