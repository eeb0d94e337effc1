"""Shared helpers for the GPU parity and invariance tests."""
import numpy as np
import pytest
import torch

# Tolerances against the fp64 oracle (per element, r = oracle value)
def tol_logits(r):
    return 2e-5 + 1e-5 * np.abs(r)


TOL_FUSED = 2e-3
TOL_BWD = 1e-3

# Parameter gradients (grad_hidden = D . W, grad_weight = D^T . h).  The pages
# give no bound for them; the target's backward bound (1e-3 absolute) applies
# to every gradient output, and on top of it an fp32-grade bound fixed before
# any measurement: 1e-4 of the sum of the absolute values of the summed terms
# (sum_j |D_ij| |W_jk|, or sum_i |D_ij| |h_ik|), plus 1e-5.  That is ten times
# the accumulated rounding of an fp32 sum of up to 2^18 terms on random data
# and far inside what one bf16 rounding of D alone would cost (up to 2^-8 of
# the same sum).
PARAM_REL = 1e-4
PARAM_ABS = 1e-5


def param_tol(scale):
    """Per-element bound for a parameter gradient whose summed terms have
    absolute sum ``scale``: both the backward bound and the fp32-grade one."""
    return np.minimum(TOL_BWD, PARAM_REL * np.asarray(scale, dtype=np.float64) + PARAM_ABS)


_ORACLE_CACHE = {}


def oracle_cached(key, fn):
    """fn() once per key per test session (full-size oracle forwards are
    shared between test modules; the key names the workload and seed)."""
    if key not in _ORACLE_CACHE:
        _ORACLE_CACHE[key] = fn()
    return _ORACLE_CACHE[key]


def oracle_logp_rows(bits, targets, mask, block_rows=64):
    """oracle.logp_selected over every row of host bf16 bits, row blocks in a
    thread pool (rows are independent: the values are those of one call)."""
    import oracle
    from oracle.parallel import map_row_blocks
    n = bits.shape[0]
    return map_row_blocks(
        lambda r0, r1: oracle.logp_selected(bits[r0:r1], targets[r0:r1],
                                            None if mask is None else mask[r0:r1]),
        n, block_rows)


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
