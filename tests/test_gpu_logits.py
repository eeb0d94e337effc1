"""GPU parity of the logits path (forward K1, backward K2) against the fp64
oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import invariant_logprob_amd as ilp
import oracle
from gpu_util import TOL_BWD, assert_close, bits16, f32bits, padded_bf16, require_gpu, tol_logits
from invariant_logprob_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    ilp.load_library()
    return d


def _run_and_compare(logits, targets, mask, what, grad=None):
    logp, lse = ilp.logp_selected(logits, targets, mask)
    torch.cuda.synchronize()
    bits = bits16(logits)
    t = targets.cpu().numpy()
    m = None if mask is None else mask.cpu().numpy()
    rlogp, rlse = oracle.logp_selected(bits, t, m)
    act = np.ones(len(t), bool) if m is None else m.astype(bool)
    assert_close(logp.cpu().numpy(), rlogp, tol_logits, f"{what} logp", act)
    assert_close(lse.cpu().numpy(), rlse, tol_logits, f"{what} lse", act)
    assert np.all(f32bits(logp).numpy()[~act] == 0) and np.all(f32bits(lse).numpy()[~act] == 0)
    if grad is not None:
        d = ilp.logp_backward(logits, targets, lse, grad, mask)
        torch.cuda.synchronize()
        rd = oracle.logp_backward(bits, t, m, lse.cpu().numpy().astype(np.float64),
                                  grad.cpu().numpy())
        assert_close(d.cpu().numpy(), rd, TOL_BWD, f"{what} dlogits")
        assert np.all(f32bits(d).numpy()[~act] == 0), "inactive rows must be +0.0"
    return logp, lse


def test_small_config_parity(dev):
    b = wl.logits_small(seed=0, device=dev)
    _run_and_compare(b.logits, b.targets, b.mask, "N=8 V=1024", grad=b.grad)


@pytest.mark.parametrize("v", [1, 2, 7, 8, 9, 15, 2047, 2049, 16384 + 3, 16384 * 3 + 8, 40001])
def test_ragged_vocab_parity(dev, v):
    n = 6
    g = torch.Generator(device=dev).manual_seed(v)
    x = (torch.randn((n, v), generator=g, device=dev) * 3).to(torch.bfloat16)
    ld = (v + 7) // 8 * 8 + 8
    logits = padded_bf16(n, v, ld, x)
    t = torch.randint(0, v, (n,), generator=g, device=dev)
    mask = torch.tensor([1, 1, 0, 1, 1, 1], dtype=torch.uint8, device=dev)
    grad = torch.randn((n,), generator=g, device=dev)
    _run_and_compare(logits, t, mask, f"V={v}", grad=grad)


def test_varlen_config_parity(dev):
    """8 packed varlen sequences, V=32000, 5% peaked rows, half argmax targets:
    one launch over all rows; the oracle checks a seeded sample of 1024 rows
    (peaked rows and the last rows included) and every padding row is +0.0."""
    b = wl.logits_varlen(seed=0, device=dev)
    logp, lse = ilp.logp_selected(b.logits, b.targets, b.mask)
    torch.cuda.synchronize()
    n = b.logits.shape[0]
    total = sum(b.seq_lens)
    peaked = torch.nonzero(b.logits.float().amax(dim=1) > 15).flatten().cpu().tolist()
    pick = torch.randperm(n, generator=torch.Generator().manual_seed(3))[:1024].tolist()
    rows = sorted(set(pick + peaked[:64] + [0, total - 1, total, n - 1]))
    idx = torch.tensor(rows, device=dev)
    sub = b.logits.index_select(0, idx)
    t = b.targets.index_select(0, idx).cpu().numpy()
    m = b.mask.index_select(0, idx).cpu().numpy()
    rlogp, rlse = oracle.logp_selected(bits16(sub), t, m)
    act = m.astype(bool)
    assert act.sum() > 900 and len(peaked) > 100
    assert_close(logp.index_select(0, idx).cpu().numpy(), rlogp, tol_logits, "varlen logp", act)
    assert_close(lse.index_select(0, idx).cpu().numpy(), rlse, tol_logits, "varlen lse", act)
    assert bool((f32bits(logp)[total:] == 0).all()) and bool((f32bits(lse)[total:] == 0).all())
    # backward on a bounded slice of rows (the oracle's dense [N, V] output)
    sl = slice(0, 96)
    lp, lse96 = ilp.logp_selected(b.logits[sl], b.targets[sl], b.mask[sl])
    d = ilp.logp_backward(b.logits[sl], b.targets[sl], lse96, b.grad[sl], b.mask[sl])
    rd = oracle.logp_backward(bits16(b.logits[sl]), b.targets[sl].cpu().numpy(),
                              b.mask[sl].cpu().numpy(), lse96.cpu().numpy(), b.grad[sl].cpu().numpy())
    assert_close(d.cpu().numpy(), rd, TOL_BWD, "varlen dlogits")


def test_large_config_sampled_rows(dev):
    """N=16384, V=151936 in one launch; rows sampled for the oracle."""
    b = wl.logits_large(seed=0, device=dev)
    logp, lse = ilp.logp_selected(b.logits, b.targets, b.mask)
    torch.cuda.synchronize()
    n = b.logits.shape[0]
    rows = sorted(set([0, 1, 255, 256, 8191, n - 2, n - 1] +
                      torch.randperm(n, generator=torch.Generator().manual_seed(5))[:40].tolist()))
    idx = torch.tensor(rows, device=dev)
    sub_bits = bits16(b.logits.index_select(0, idx))
    t = b.targets.index_select(0, idx).cpu().numpy()
    m = b.mask.index_select(0, idx).cpu().numpy()
    rlogp, rlse = oracle.logp_selected(sub_bits, t, m)
    act = m.astype(bool)
    assert_close(logp.index_select(0, idx).cpu().numpy(), rlogp, tol_logits, "large logp", act)
    assert_close(lse.index_select(0, idx).cpu().numpy(), rlse, tol_logits, "large lse", act)
    inactive = (b.mask == 0)
    assert int(inactive.sum()) == 2458
    assert bool((f32bits(logp)[inactive.cpu()] == 0).all())
    # backward at full size, sampled rows
    d = ilp.logp_backward(b.logits, b.targets, lse, b.grad, b.mask)
    torch.cuda.synchronize()
    rd = oracle.logp_backward(sub_bits, t, m, lse.index_select(0, idx).cpu().numpy(),
                              b.grad.index_select(0, idx).cpu().numpy())
    assert_close(d.index_select(0, idx).cpu().numpy(), rd, TOL_BWD, "large dlogits")
    # property at any size: each active row of dlogits sums to ~0
    rs = d[:4096].double().sum(dim=1).cpu().numpy()
    act4 = b.mask[:4096].cpu().numpy().astype(bool)
    assert np.max(np.abs(rs[act4])) < 1e-3


def test_closed_forms(dev):
    for v in (1, 3, 1024, 32000, 151936):
        ld = (v + 7) // 8 * 8
        x = padded_bf16(3, v, ld, torch.full((3, v), 2.5, dtype=torch.bfloat16, device=dev))
        t = torch.tensor([0, v // 2, v - 1], device=dev)
        logp, lse = ilp.logp_selected(x, t)
        ref = -math.log(v)
        assert np.allclose(logp.cpu().numpy(), ref, atol=2e-5 + 1e-5 * abs(ref), rtol=0), (v, logp)
        if v == 1:
            assert bool((logp == 0).all())
    # peaked row: -ln(1 + (V-1) e^-L)
    v, L = 32000, 20.0
    x = torch.zeros((1, v), dtype=torch.bfloat16, device=dev)
    x[0, 123] = L
    logp, _ = ilp.logp_selected(x, torch.tensor([123], device=dev))
    ref = -math.log1p((v - 1) * math.exp(-L))
    assert abs(float(logp[0]) - ref) <= 2e-5 + 1e-5 * abs(ref)


def test_nonfinite_and_invalid_targets(dev):
    v = 3000
    x = torch.zeros((4, v), dtype=torch.float32, device=dev)
    x[0, ::2] = float("-inf")          # -inf entries contribute nothing
    x[1, 7] = float("inf")             # +inf -> NaN
    x[2, 9] = float("nan")             # NaN -> NaN
    logits = x.to(torch.bfloat16)
    t = torch.tensor([1, 0, 0, v + 5], device=dev)   # row 3: invalid target on an active row
    logp, lse = ilp.logp_selected(logits, t)
    lp = logp.cpu().numpy()
    assert abs(lp[0] + math.log(v // 2)) <= 2e-5 + 1e-5 * math.log(v)
    assert np.isnan(lp[1]) and np.isnan(lp[2]) and np.isnan(lp[3])
    d = ilp.logp_backward(logits, t, lse, torch.ones(4, device=dev))
    assert bool(torch.isnan(d[3]).all())
    # masked row with an invalid target is fine and exactly zero
    mask = torch.tensor([1, 1, 1, 0], dtype=torch.uint8, device=dev)
    logp2, _ = ilp.logp_selected(logits, t, mask)
    assert int(f32bits(logp2)[3]) == 0


def test_run_to_run_determinism(dev):
    b = wl.logits_varlen(seed=1, device=dev)
    outs = [ilp.logp_selected(b.logits, b.targets, b.mask) for _ in range(3)]
    d = [ilp.logp_backward(b.logits[:64], b.targets[:64], outs[0][1][:64], b.grad[:64],
                           b.mask[:64]) for _ in range(3)]
    for o in outs[1:]:
        assert torch.equal(f32bits(o[0]), f32bits(outs[0][0]))
        assert torch.equal(f32bits(o[1]), f32bits(outs[0][1]))
    for x in d[1:]:
        assert torch.equal(f32bits(x), f32bits(d[0]))


def test_empty_and_errors(dev):
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev)
    t = torch.zeros((0,), dtype=torch.int64, device=dev)
    lp, lse = ilp.logp_selected(x, t)
    assert lp.numel() == 0
    # a row stride that is not a multiple of 8 elements is refused, not peeled
    y = torch.zeros((4, 100), dtype=torch.bfloat16, device=dev).as_strided((4, 99), (99, 1))
    with pytest.raises(ilp.RlkError) as e:
        ilp.logp_selected(y, torch.zeros(4, dtype=torch.int64, device=dev))
    assert e.value.status == 2


def test_autograd_wrapper(dev):
    from invariant_logprob_amd._binding import SelectedLogprob
    b = wl.logits_small(seed=3, device=dev)
    x = b.logits.clone().requires_grad_(True)
    lp = SelectedLogprob.apply(x, b.targets, b.mask)
    (lp * b.grad).sum().backward()
    _, lse = ilp.logp_selected(b.logits, b.targets, b.mask)
    d = ilp.logp_backward(b.logits, b.targets, lse, b.grad, b.mask)
    assert torch.equal(x.grad.float(), d.to(torch.bfloat16).float())
