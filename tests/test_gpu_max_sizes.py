"""GPU parity at the size limits the C ABI accepts, against the fp64 oracle on
sampled rows or entries:

* the largest vocabulary, V = 2^28 (one row holds 512 MB of bf16 logits);
* more than 2^31 logits elements in one call, so that any 32-bit element
  offset would wrap;
* a fused vocabulary of 2^21 + 7 entries (8193 vocabulary tiles, a ragged
  last one);
* the largest fused leading dimension, H = ld = 2^22 - 8: a 256-row slab of W
  spans 2^31 - 4096 bytes, the edge of the tiles' 32-bit buffer ranges.

Tolerances are the same as at ordinary sizes."""
import numpy as np
import pytest
import torch

import invariant_logprob_amd as ilp
import oracle
from gpu_util import TOL_BWD, TOL_FUSED, assert_close, bits16, f32bits, require_gpu, tol_logits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    ilp.load_library()
    return d


def _randn_bf16(shape, sigma, seed, dev):
    g = torch.Generator(device=dev).manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    flat = out.view(-1)
    step = 1 << 26
    for i in range(0, flat.numel(), step):
        n = min(step, flat.numel() - i)
        flat[i:i + n] = (torch.randn(n, generator=g, device=dev) * sigma).to(torch.bfloat16)
    return out


def test_largest_vocabulary_row(dev):
    v = 1 << 28
    x = _randn_bf16((2, v), 3.0, 101, dev)
    t = torch.tensor([12345, v - 1], dtype=torch.int64, device=dev)
    logp, lse = ilp.logp_selected(x, t)
    g = torch.tensor([0.5, -2.0], device=dev)
    d = ilp.logp_backward(x, t, lse, g)
    torch.cuda.synchronize()
    bits = bits16(x)
    rlogp, rlse = oracle.logp_selected(bits, t.cpu().numpy(), block_rows=1)
    assert_close(logp.cpu().numpy(), rlogp, tol_logits, "V=2^28 logp")
    assert_close(lse.cpu().numpy(), rlse, tol_logits, "V=2^28 lse")
    # sampled gradient entries, including both targets and the row ends
    cols = np.unique(np.concatenate([
        np.random.default_rng(5).integers(0, v, 2000), [0, 1, 12345, v - 2, v - 1]]))
    xs = oracle.bf16_to_f64(bits[:, cols])
    tl = t.cpu().numpy()
    ci = torch.from_numpy(cols).to(dev)
    for r in range(2):
        onehot = (cols == tl[r]).astype(np.float64)
        rd = float(g[r]) * (onehot - np.exp(xs[r] - rlse[r]))   # the oracle's own lse
        assert_close(d[r].index_select(0, ci).cpu().numpy(), rd, TOL_BWD, f"V=2^28 dlogits row {r}")


def test_more_than_2g_elements(dev):
    n, v = (1 << 21) + 3, 1032          # 2.16e9 elements, ld = V
    x = _randn_bf16((n, v), 4.0, 102, dev)
    g = torch.Generator(device=dev).manual_seed(103)
    t = torch.randint(0, v, (n,), generator=g, device=dev)
    mask = torch.ones(n, dtype=torch.uint8, device=dev)
    mask[::7] = 0
    grad = torch.randn(n, generator=g, device=dev)
    logp, lse = ilp.logp_selected(x, t, mask)
    d = ilp.logp_backward(x, t, lse, grad, mask)
    torch.cuda.synchronize()
    rows = [0, 1, 2, 1 << 20, (1 << 21) - 1, n - 3, n - 2, n - 1]
    idx = torch.tensor(rows, device=dev)
    sb = bits16(x.index_select(0, idx))
    st = t.index_select(0, idx).cpu().numpy()
    sm = mask.index_select(0, idx).cpu().numpy()
    rlogp, rlse = oracle.logp_selected(sb, st, sm)
    act = sm.astype(bool)
    assert_close(logp.index_select(0, idx).cpu().numpy(), rlogp, tol_logits, ">2^31 logp", act)
    assert_close(lse.index_select(0, idx).cpu().numpy(), rlse, tol_logits, ">2^31 lse", act)
    rd = oracle.logp_backward(sb, st, sm, rlse, grad.index_select(0, idx).cpu().numpy())
    assert_close(d.index_select(0, idx).cpu().numpy(), rd, TOL_BWD, ">2^31 dlogits")
    last_masked = (n - 1) // 7 * 7
    assert bool((f32bits(d[last_masked:last_masked + 1]) == 0).all())
    assert bool((f32bits(logp[::7]) == 0).all())


def test_fused_large_vocabulary(dev):
    n, v, h = 40, (1 << 21) + 7, 64
    hid = _randn_bf16((n, h), 1.0, 104, dev)
    w = _randn_bf16((v, h), 0.05, 105, dev)
    g = torch.Generator(device=dev).manual_seed(106)
    t = torch.randint(0, v, (n,), generator=g, device=dev)
    t[0] = v - 1
    grad = torch.randn(n, generator=g, device=dev)
    logp, lse = ilp.linear_logp(hid, w, t)
    d = ilp.linear_logp_backward(hid, w, t, lse, grad)
    torch.cuda.synchronize()
    hb, wb = bits16(hid), bits16(w)
    tt = t.cpu().numpy()
    rlogp, rlse = oracle.linear_logp(hb, wb, tt)
    assert_close(logp.cpu().numpy(), rlogp, TOL_FUSED, "V=2^21+7 fused logp")
    assert_close(lse.cpu().numpy(), rlse, TOL_FUSED, "V=2^21+7 fused lse")
    rows = [0, 17, n - 1]
    rd = oracle.linear_logp_backward(hb[rows], wb, tt[rows], None, rlse[rows],
                                     grad.cpu().numpy()[rows])
    assert_close(d.cpu().numpy()[rows], rd, TOL_BWD, "V=2^21+7 fused dlogits")


def test_fused_largest_leading_dimension(dev):
    n, v, h = 3, 260, (1 << 22) - 8
    hid = _randn_bf16((n, h), 1.0, 107, dev)
    w = _randn_bf16((v, h), 0.0005, 108, dev)
    t = torch.tensor([0, 259, 256], dtype=torch.int64, device=dev)
    logp, lse = ilp.linear_logp(hid, w, t)
    grad = torch.tensor([1.0, -0.5, 2.0], device=dev)
    d = ilp.linear_logp_backward(hid, w, t, lse, grad)
    torch.cuda.synchronize()
    hb, wb = bits16(hid), bits16(w)
    rlogp, rlse = oracle.linear_logp(hb, wb, t.cpu().numpy())
    assert_close(logp.cpu().numpy(), rlogp, TOL_FUSED, "H=2^22-8 fused logp")
    assert_close(lse.cpu().numpy(), rlse, TOL_FUSED, "H=2^22-8 fused lse")
    rd = oracle.linear_logp_backward(hb, wb, t.cpu().numpy(), None, rlse, grad.cpu().numpy())
    assert_close(d.cpu().numpy(), rd, TOL_BWD, "H=2^22-8 fused dlogits")
