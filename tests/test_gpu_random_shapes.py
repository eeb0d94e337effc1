"""A seeded sweep of ragged shapes and strides through every path, against
the fp64 oracle: logits forward and backward, fused forward, recomputing and
kept-logits backward, and the parameter gradients.  Each case draws N, V, H,
a padded leading dimension (its padding filled with NaN, which must never be
read), a mask and a logit scale; two of its rows are then recomputed alone,
and for the fused path a random contiguous run of 2..160 rows as its own
batch, and must give the same bits (the I-relation under population change).
Gradient references are the oracle's, from the inputs alone (its own lse)."""
import numpy as np
import pytest
import torch

import invariant_logprob_amd as ilp
import oracle
from gpu_util import (TOL_BWD, TOL_FUSED, assert_close, bits16, f32bits, param_tol, require_gpu,
                      tol_logits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    ilp.load_library()
    return d


def _padded(rows, cols, ld, scale, gen, dev):
    """[rows, cols] bf16 view of a [rows, ld] buffer whose padding is NaN."""
    buf = torch.full((rows, ld), float("nan"), dtype=torch.bfloat16, device=dev)
    buf[:, :cols] = (torch.randn((rows, cols), generator=gen, device=dev) * scale).to(torch.bfloat16)
    return buf[:, :cols]


@pytest.mark.parametrize("seed", range(12))
def test_logits_path_random_shape(dev, seed):
    r = np.random.default_rng(1000 + seed)
    n = int(r.integers(1, 700))
    v = int(r.integers(1, 5000))
    ld = (v + 7) // 8 * 8 + 8 * int(r.integers(0, 4))
    scale = float(r.choice([1.0, 3.0, 6.0]))
    gen = torch.Generator(device=dev).manual_seed(seed)
    x = _padded(n, v, ld, scale, gen, dev)
    t = torch.randint(0, v, (n,), generator=gen, device=dev)
    mask = (torch.rand(n, generator=gen, device=dev) > float(r.uniform(0.0, 0.4))).to(torch.uint8)
    g = torch.randn(n, generator=gen, device=dev)
    logp, lse = ilp.logp_selected(x, t, mask)
    d = ilp.logp_backward(x, t, lse, g, mask)
    torch.cuda.synchronize()
    xb = bits16(x)
    tt, mm = t.cpu().numpy(), mask.cpu().numpy()
    rlogp, rlse = oracle.logp_selected(xb, tt, mm)
    act = mm.astype(bool)
    what = f"seed {seed}: {n}x{v} ld {ld}"
    assert_close(logp.cpu().numpy(), rlogp, tol_logits, f"logp {what}", act)
    assert_close(lse.cpu().numpy(), rlse, tol_logits, f"lse {what}", act)
    rd = oracle.logp_backward(xb, tt, mm, rlse, g.cpu().numpy())
    assert_close(d.cpu().numpy(), rd, TOL_BWD, f"dlogits {what}")
    assert bool((f32bits(logp)[torch.from_numpy(~act)] == 0).all())
    for i in r.choice(n, size=min(2, n), replace=False):
        i = int(i)
        lp1, ls1 = ilp.logp_selected(x[i:i + 1], t[i:i + 1], mask[i:i + 1])
        d1 = ilp.logp_backward(x[i:i + 1], t[i:i + 1], ls1, g[i:i + 1], mask[i:i + 1])
        torch.cuda.synchronize()
        assert torch.equal(f32bits(lp1), f32bits(logp[i:i + 1])), (what, i)
        assert torch.equal(f32bits(ls1), f32bits(lse[i:i + 1])), (what, i)
        assert torch.equal(f32bits(d1), f32bits(d[i:i + 1])), (what, i)


@pytest.mark.parametrize("seed", range(10))
def test_fused_path_random_shape(dev, seed):
    r = np.random.default_rng(2000 + seed)
    n = int(r.integers(1, 600))
    v = int(r.integers(1, 3000))
    h = 8 * int(r.integers(1, 80))
    ldh = h + 8 * int(r.integers(0, 3))
    ldw = h + 8 * int(r.integers(0, 3))
    gen = torch.Generator(device=dev).manual_seed(100 + seed)
    hid = _padded(n, h, ldh, 1.0, gen, dev)
    w = _padded(v, h, ldw, float(r.choice([0.02, 0.05, 0.2])), gen, dev)
    t = torch.randint(0, v, (n,), generator=gen, device=dev)
    mask = (torch.rand(n, generator=gen, device=dev) > float(r.uniform(0.0, 0.4))).to(torch.uint8)
    g = torch.randn(n, generator=gen, device=dev)
    what = f"seed {seed}: {n}x{v}x{h} ld {ldh}/{ldw}"

    logp, lse = ilp.linear_logp(hid, w, t, mask)
    d = ilp.linear_logp_backward(hid, w, t, lse, g, mask)
    klogp, klse, z = ilp.linear_logp_with_logits(hid, w, t, mask)
    dk = ilp.logp_backward(z, t, klse, g, mask)
    gh, gw = ilp.linear_logp_param_grads(hid, w, t, lse, g, mask)
    gh2, gw2 = ilp.linear_logp_param_grads(hid, w, t, klse, g, mask, logits=z)
    torch.cuda.synchronize()

    hb, wb = bits16(hid), bits16(w)
    tt, mm = t.cpu().numpy(), mask.cpu().numpy()
    act = mm.astype(bool)
    rlogp, rlse = oracle.linear_logp(hb, wb, tt, mm)
    assert_close(logp.cpu().numpy(), rlogp, TOL_FUSED, f"fused logp {what}", act)
    assert_close(lse.cpu().numpy(), rlse, TOL_FUSED, f"fused lse {what}", act)
    gg = g.cpu().numpy()
    rd = oracle.linear_logp_backward(hb, wb, tt, mm, rlse, gg)
    assert_close(d.cpu().numpy(), rd, TOL_BWD, f"fused dlogits {what}")
    # the kept-logits route gives the same bits as the recomputing one
    for a, b, nm in ((klogp, logp, "logp"), (klse, lse, "lse"), (dk, d, "dlogits"),
                     (gh2, gh, "grad_hidden"), (gw2, gw, "grad_weight")):
        assert torch.equal(f32bits(a), f32bits(b)), (what, nm)
    rgh, rgw = oracle.linear_param_grads(hb, wb, tt, mm, rlse, gg)
    d_abs = np.abs(rd)
    assert_close(gh.cpu().numpy(), rgh, param_tol(d_abs @ np.abs(oracle.bf16_to_f64(wb))),
                 f"grad_hidden {what}")
    assert_close(gw.cpu().numpy(), rgw, param_tol(d_abs.T @ np.abs(oracle.bf16_to_f64(hb))),
                 f"grad_weight {what}")
    for i in r.choice(n, size=min(2, n), replace=False):
        i = int(i)
        lp1, ls1 = ilp.linear_logp(hid[i:i + 1], w, t[i:i + 1], mask[i:i + 1])
        d1 = ilp.linear_logp_backward(hid[i:i + 1], w, t[i:i + 1], ls1, g[i:i + 1], mask[i:i + 1])
        gh1, _ = ilp.linear_logp_param_grads(hid[i:i + 1], w, t[i:i + 1], ls1, g[i:i + 1],
                                             mask[i:i + 1], want_weight=False)
        torch.cuda.synchronize()
        assert torch.equal(f32bits(lp1), f32bits(logp[i:i + 1])), (what, i)
        assert torch.equal(f32bits(ls1), f32bits(lse[i:i + 1])), (what, i)
        assert torch.equal(f32bits(d1), f32bits(d[i:i + 1])), (what, i)
        assert torch.equal(f32bits(gh1), f32bits(gh[i:i + 1])), (what, i)
    # a random contiguous sub-batch of 2..160 rows (any launch form of the fused kernels)
    if n >= 2:
        k = int(r.integers(2, min(n, 160) + 1))
        s0 = int(r.integers(0, n - k + 1))
        sl = slice(s0, s0 + k)
        lpk, lsk = ilp.linear_logp(hid[sl], w, t[sl], mask[sl])
        dkk = ilp.linear_logp_backward(hid[sl], w, t[sl], lsk, g[sl], mask[sl])
        torch.cuda.synchronize()
        assert torch.equal(f32bits(lpk), f32bits(logp[sl])), (what, s0, k)
        assert torch.equal(f32bits(lsk), f32bits(lse[sl])), (what, s0, k)
        assert torch.equal(f32bits(dkk), f32bits(d[sl])), (what, s0, k)
