"""GPU checks of the fused forward that keeps its fp32 logits
(rlk_linear_logp_with_logits) and of the backward from fp32 logits
(rlk_logp_backward_f32), through the C ABI.

The pages' fused backward is onehot minus softmax scaled by the upstream
gradient, with the logits batch-invariant (page "[WS1 Test] #154 dtype pin +
#152 KV path + #153 bwd invariance + #150 chain gate", section "Workstream 3 -
#153").  Keeping the logits must change nothing but the cost: logp and lse
equal linear_logp's bit for bit, and the gradient equals the recomputing fused
backward's bit for bit.  The kept logits themselves are checked against the
fp64 oracle within the bound of an fp32 sum of H exact products."""
import numpy as np
import pytest
import torch

import invariant_logprob_amd as ilp
import oracle
from gpu_util import TOL_BWD, assert_close, bits16, f32bits, require_gpu
from invariant_logprob_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    ilp.load_library()
    return d


def _bits_equal(a, b):
    return bool(torch.equal(f32bits(a), f32bits(b)))


def _logits_bound(hidden, weight):
    """|fp32 sum of H exact products - exact sum| <= H 2^-24 sum_k |h_k w_k|."""
    h = np.abs(oracle.bf16_to_f64(bits16(hidden)))
    w = np.abs(oracle.bf16_to_f64(bits16(weight)))
    return hidden.shape[1] * 2.0 ** -24 * (h @ w.T) + 1e-30


def _padded_f32(n, v, ld, dev):
    """[n, v] view of an [n, ld] fp32 buffer whose padding holds a NaN sentinel."""
    buf = torch.full((n, ld), float("nan"), dtype=torch.float32, device=dev)
    return buf, buf[:, :v]


@pytest.mark.parametrize("n,v,h", [(1, 256, 64), (37, 1000, 136), (300, 2600, 512), (257, 513, 8)])
def test_small_parity_and_bits(dev, n, v, h):
    b = wl.fused_batch(n, v, h, seed=7 * n + v + h, device=dev, w_sigma=0.05, n_masked=n // 10)
    ld = (v + 3) // 4 * 4 + 8
    zbuf, zview = _padded_f32(n, v, ld, dev)
    pad_before = f32bits(zbuf[:, v:]).clone()
    logp, lse, z = ilp.linear_logp_with_logits(b.hidden, b.weight, b.targets, b.mask, logits=zview)
    logp0, lse0 = ilp.linear_logp(b.hidden, b.weight, b.targets, b.mask)
    torch.cuda.synchronize()
    assert _bits_equal(logp, logp0) and _bits_equal(lse, lse0)
    # the kept logits: every row (masked ones too), within the fp32 summation bound
    rz = oracle.linear_logits(bits16(b.hidden), bits16(b.weight))
    err = np.abs(z.cpu().numpy().astype(np.float64) - rz) - _logits_bound(b.hidden, b.weight)
    assert err.max() <= 0, f"logits outside the summation bound by {err.max()}"
    assert torch.equal(f32bits(zbuf[:, v:]), pad_before), "columns >= V were written"
    # the backward from them equals the recomputing fused backward bit for bit
    d_re = ilp.linear_logp_backward(b.hidden, b.weight, b.targets, lse, b.grad, b.mask)
    dbuf, dview = _padded_f32(n, v, ld, dev)
    d = ilp.logp_backward(z, b.targets, lse, b.grad, b.mask, out=dview)
    torch.cuda.synchronize()
    assert _bits_equal(d, d_re)
    assert bool(torch.isnan(dbuf[:, v:]).all()), "columns >= V of the gradient were written"
    act = b.mask.cpu().numpy().astype(bool)
    _, rlse = oracle.linear_logp(bits16(b.hidden), bits16(b.weight), b.targets.cpu().numpy(),
                                 act.astype(np.uint8))
    rd = oracle.linear_logp_backward(bits16(b.hidden), bits16(b.weight), b.targets.cpu().numpy(),
                                     act.astype(np.uint8), rlse, b.grad.cpu().numpy())
    assert_close(d.cpu().numpy(), rd, TOL_BWD, f"dlogits from kept logits {n}x{v}x{h} (end to end)")
    assert bool((f32bits(d)[~torch.from_numpy(act)] == 0).all()), "masked rows not +0.0"
    # in place: the gradient overwrites the logits
    z2 = zbuf.clone()[:, :v]
    d2 = ilp.logp_backward(z2, b.targets, lse, b.grad, b.mask, out=z2)
    torch.cuda.synchronize()
    assert d2.data_ptr() == z2.data_ptr() and _bits_equal(d2, d_re)


def test_invalid_target_and_masked_rows(dev):
    n, v, h = 40, 1000, 64
    b = wl.fused_batch(n, v, h, seed=11, device=dev, w_sigma=0.05)
    t = b.targets.clone()
    t[3] = v          # active, out of range
    t[4] = -1         # active, out of range
    mask = torch.ones(n, dtype=torch.uint8, device=dev)
    mask[5] = 0       # masked: its target is never read
    t[5] = 10 ** 9
    logp, lse, z = ilp.linear_logp_with_logits(b.hidden, b.weight, t, mask)
    d = ilp.logp_backward(z, t, lse, b.grad, mask)
    d_re = ilp.linear_logp_backward(b.hidden, b.weight, t, lse, b.grad, mask)
    torch.cuda.synchronize()
    assert bool(torch.isnan(d[3]).all()) and bool(torch.isnan(d[4]).all())
    assert bool((f32bits(d[5]) == 0).all())
    assert bool(torch.isnan(logp[3])) and int(f32bits(logp[5:6])[0]) == 0
    keep = [i for i in range(n) if i not in (3, 4)]
    assert _bits_equal(d[keep], d_re[keep])


def test_row_invariance(dev):
    """A row's kept logits and gradient do not depend on the batch around it:
    single rows, a permuted subset and a ragged slice against the full batch."""
    n, v, h = 300, 1300, 136
    b = wl.fused_batch(n, v, h, seed=13, device=dev, w_sigma=0.05, n_masked=20)
    logp, lse, z = ilp.linear_logp_with_logits(b.hidden, b.weight, b.targets, b.mask)
    d = ilp.logp_backward(z, b.targets, lse, b.grad, b.mask)
    for r in (0, 1, 255, 256, 299):
        lp1, ls1, z1 = ilp.linear_logp_with_logits(b.hidden[r:r + 1], b.weight, b.targets[r:r + 1],
                                                   b.mask[r:r + 1])
        d1 = ilp.logp_backward(z1, b.targets[r:r + 1], ls1, b.grad[r:r + 1], b.mask[r:r + 1])
        assert _bits_equal(z1, z[r:r + 1]) and _bits_equal(lp1, logp[r:r + 1]), r
        assert _bits_equal(d1, d[r:r + 1]), r
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(3))[:77].to(dev)
    lpp, lsp, zp = ilp.linear_logp_with_logits(b.hidden.index_select(0, perm).contiguous(), b.weight,
                                               b.targets.index_select(0, perm),
                                               b.mask.index_select(0, perm))
    dp = ilp.logp_backward(zp, b.targets.index_select(0, perm), lsp, b.grad.index_select(0, perm),
                           b.mask.index_select(0, perm))
    assert _bits_equal(zp, z.index_select(0, perm)) and _bits_equal(dp, d.index_select(0, perm))
    lps, lss, zs = ilp.linear_logp_with_logits(b.hidden[17:290], b.weight, b.targets[17:290],
                                               b.mask[17:290])
    assert _bits_equal(zs, z[17:290]) and _bits_equal(lps, logp[17:290])


def test_fwd_bwd_full_size(dev):
    """hidden [2048, 5120], W [151936, 5120], upstream grad N(0, 1): the kept
    logits' gradient equals the recomputing fused backward's over the whole
    [N, V] output; sampled rows of the kept logits against the oracle."""
    b = wl.fused_bwd(seed=0, device=dev)
    logp0, lse0 = ilp.linear_logp(b.hidden, b.weight, b.targets, b.mask)
    d_re = ilp.linear_logp_backward(b.hidden, b.weight, b.targets, lse0, b.grad, b.mask)
    logp, lse, z = ilp.linear_logp_with_logits(b.hidden, b.weight, b.targets, b.mask)
    torch.cuda.synchronize()
    assert _bits_equal(logp, logp0) and _bits_equal(lse, lse0)
    rows = [0, 777, 2047]
    idx = torch.tensor(rows, device=dev)
    sub_h = b.hidden.index_select(0, idx)
    rz = oracle.linear_logits(bits16(sub_h), bits16(b.weight))
    err = np.abs(z.index_select(0, idx).cpu().numpy().astype(np.float64) - rz) - \
        _logits_bound(sub_h, b.weight)
    assert err.max() <= 0, f"logits outside the summation bound by {err.max()}"
    d = ilp.logp_backward(z, b.targets, lse, b.grad, b.mask, out=z)   # in place
    torch.cuda.synchronize()
    assert _bits_equal(d, d_re)


def test_empty_batch(dev):
    w = torch.randn((300, 64), device=dev).to(torch.bfloat16)
    h = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    t = torch.empty(0, dtype=torch.int64, device=dev)
    logp, lse, z = ilp.linear_logp_with_logits(h, w, t)
    assert logp.shape == (0,) and z.shape == (0, 300)
    d = ilp.logp_backward(z, t, lse, torch.empty(0, device=dev))
    assert d.shape == (0, 300)


def test_binding_refuses_rows_its_storage_does_not_hold(dev):
    """Rows are read in whole aligned groups up to the leading dimension; a
    lone row whose storage ends before that is refused, not over-read."""
    x = torch.randn((1, 1001), device=dev).to(torch.bfloat16)
    t = torch.zeros(1, dtype=torch.int64, device=dev)
    with pytest.raises(ValueError):
        ilp.logp_selected(x, t)
    z = torch.randn((1, 1001), device=dev)
    with pytest.raises(ValueError):
        ilp.logp_backward(z, t, torch.zeros(1, device=dev), torch.ones(1, device=dev))
    # the same row inside padded storage is fine
    xp = torch.randn((1, 1008), device=dev).to(torch.bfloat16)[:, :1001]
    ilp.logp_selected(xp, t)


@pytest.mark.parametrize("n,v,h", [(33, 1000, 256), (300, 17000, 136), (257, 513, 8)])
def test_param_grads_from_kept_logits(dev, n, v, h):
    """Parameter gradients from the kept logits equal the recomputing path's
    bit for bit: several vocabulary chunks with a ragged last one, masked rows
    and one active row with an invalid target (NaN in the same places)."""
    b = wl.fused_batch(n, v, h, seed=5 * n + v, device=dev, w_sigma=0.05, n_masked=n // 10)
    t = b.targets.clone()
    t[1] = v
    b.mask[1] = 1
    logp, lse, z = ilp.linear_logp_with_logits(b.hidden, b.weight, t, b.mask)
    gh0, gw0 = ilp.linear_logp_param_grads(b.hidden, b.weight, t, lse, b.grad, b.mask)
    gh1, gw1 = ilp.linear_logp_param_grads(b.hidden, b.weight, t, lse, b.grad, b.mask, logits=z)
    torch.cuda.synchronize()
    assert _bits_equal(gh1, gh0) and _bits_equal(gw1, gw0)
    assert bool(torch.isnan(gh1[1]).all())
    # without the invalid row: finite, and still equal
    t[1] = 0
    logp, lse, z = ilp.linear_logp_with_logits(b.hidden, b.weight, t, b.mask)
    gh0, gw0 = ilp.linear_logp_param_grads(b.hidden, b.weight, t, lse, b.grad, b.mask)
    gh1, gw1 = ilp.linear_logp_param_grads(b.hidden, b.weight, t, lse, b.grad, b.mask, logits=z,
                                           want_hidden=False)
    torch.cuda.synchronize()
    assert gh1 is None and _bits_equal(gw1, gw0) and bool(torch.isfinite(gw1).all())


def test_param_grads_from_kept_logits_full_size(dev):
    """hidden [2048, 5120], W [151936, 5120]: both gradients from the kept
    logits equal the recomputing path's over the whole outputs."""
    b = wl.fused_bwd(seed=0, device=dev)
    logp, lse, z = ilp.linear_logp_with_logits(b.hidden, b.weight, b.targets, b.mask)
    gh0, gw0 = ilp.linear_logp_param_grads(b.hidden, b.weight, b.targets, lse, b.grad, b.mask)
    torch.cuda.synchronize()
    gh1, gw1 = ilp.linear_logp_param_grads(b.hidden, b.weight, b.targets, lse, b.grad, b.mask,
                                           logits=z)
    torch.cuda.synchronize()
    assert _bits_equal(gh1, gh0)
    assert _bits_equal(gw1, gw0)
