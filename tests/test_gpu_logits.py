"""GPU parity of the logits path (forward K1, backward K2) against the fp64
oracle, through the C ABI.

Gradient references are end to end: the oracle's gradient of the whole
definition from the bf16 logits, targets, mask and upstream gradient alone
(its own log-sum-exp), never a value the GPU produced.  One separately named
unit check feeds the kernel's lse to the oracle's backward, to isolate K2."""
import math

import numpy as np
import pytest
import torch

import invariant_logprob_amd as ilp
import oracle
from gpu_util import (TOL_BWD, assert_close, bits16, f32bits, oracle_logp_rows, padded_bf16,
                      require_gpu, tol_logits)
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
        rd = oracle.logp_backward(bits, t, m, rlse, grad.cpu().numpy())
        assert_close(d.cpu().numpy(), rd, TOL_BWD, f"{what} dlogits (end to end)")
        assert np.all(f32bits(d).numpy()[~act] == 0), "inactive rows must be +0.0"
    return logp, lse


def test_small_config_parity(dev):
    b = wl.logits_small(seed=0, device=dev)
    _run_and_compare(b.logits, b.targets, b.mask, "N=8 V=1024", grad=b.grad)


@pytest.mark.parametrize("v", [1, 2, 7, 8, 9, 15, 2047, 2049, 16384 + 3, 32768, 32768 + 8, 16384 * 3 + 8, 40001])
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
    """8 packed varlen sequences, V=32000, 5% peaked rows, half argmax targets,
    in one launch: logp and lse of every row against the oracle (all active
    rows, over 4000 of them; more than 100 peaked), every padding row +0.0;
    dlogits of the first 96 rows and of 32 peaked rows, element by element,
    against the oracle's own gradient."""
    b = wl.logits_varlen(seed=0, device=dev)
    logp, lse = ilp.logp_selected(b.logits, b.targets, b.mask)
    d = ilp.logp_backward(b.logits, b.targets, lse, b.grad, b.mask)
    torch.cuda.synchronize()
    total = sum(b.seq_lens)
    peaked = torch.nonzero(b.logits.float().amax(dim=1) > 15).flatten().cpu().tolist()
    bits = bits16(b.logits)
    t = b.targets.cpu().numpy()
    m = b.mask.cpu().numpy()
    rlogp, rlse = oracle_logp_rows(bits, t, m)
    act = m.astype(bool)
    assert act.sum() == total and act.sum() > 4000 and len(peaked) > 100
    assert_close(logp.cpu().numpy(), rlogp, tol_logits, "varlen logp (all rows)", act)
    assert_close(lse.cpu().numpy(), rlse, tol_logits, "varlen lse (all rows)", act)
    assert bool((f32bits(logp)[total:] == 0).all()) and bool((f32bits(lse)[total:] == 0).all())
    rows = sorted(set(range(96)) | set(peaked[:32]))
    idx = torch.tensor(rows, device=dev)
    rd = oracle.logp_backward(bits[rows], t[rows], m[rows], None, b.grad[idx].cpu().numpy())
    assert_close(d.index_select(0, idx).cpu().numpy(), rd, TOL_BWD, "varlen dlogits (end to end)")


def test_large_config_all_rows(dev):
    """N=16384, V=151936 in one launch: logp and lse of all 13926 active rows
    against the oracle (run over row blocks in a thread pool), all 2458 masked
    rows +0.0; dlogits of 64 whole active rows (the first and last rows of
    several 256-row spans among them) element by element against the
    oracle's own gradient, 8 masked rows all +0.0, and every active row of
    the first 4096 summing to ~0."""
    b = wl.logits_large(seed=0, device=dev)
    logp, lse = ilp.logp_selected(b.logits, b.targets, b.mask)
    d = ilp.logp_backward(b.logits, b.targets, lse, b.grad, b.mask)
    torch.cuda.synchronize()
    n = b.logits.shape[0]
    bits = bits16(b.logits)
    t = b.targets.cpu().numpy()
    m = b.mask.cpu().numpy()
    act = m.astype(bool)
    assert int(act.sum()) == 13926 and int((~act).sum()) == 2458
    rlogp, rlse = oracle_logp_rows(bits, t, m)
    assert_close(logp.cpu().numpy(), rlogp, tol_logits, "large logp (all 13926 active rows)", act)
    assert_close(lse.cpu().numpy(), rlse, tol_logits, "large lse (all 13926 active rows)", act)
    assert bool((f32bits(logp)[~torch.from_numpy(act)] == 0).all())
    assert bool((f32bits(lse)[~torch.from_numpy(act)] == 0).all())
    active_rows = np.nonzero(act)[0]
    edge = [int(r) for r in active_rows[[0, 1, -2, -1]]]
    near = [int(active_rows[np.searchsorted(active_rows, k)]) for k in (255, 256, 8191, 8192)]
    pick = torch.randperm(active_rows.size, generator=torch.Generator().manual_seed(5)).tolist()
    rows = sorted(set(edge + near))
    for k in pick:
        if len(rows) == 64:
            break
        if int(active_rows[k]) not in rows:
            rows = sorted(rows + [int(active_rows[k])])
    assert len(rows) == 64
    idx = torch.tensor(rows, device=dev)
    rd = oracle.logp_backward(bits[rows], t[rows], m[rows], rlse[rows], b.grad[idx].cpu().numpy())
    assert_close(d.index_select(0, idx).cpu().numpy(), rd, TOL_BWD,
                 "large dlogits (64 whole rows, end to end)")
    masked = torch.tensor(np.nonzero(~act)[0][:8], device=dev)
    assert bool((f32bits(d.index_select(0, masked)) == 0).all())
    # property at any size: each active row of dlogits sums to ~0
    rs = d[:4096].double().sum(dim=1).cpu().numpy()
    assert np.max(np.abs(rs[act[:4096]])) < 1e-3


def test_k2_unit_check_with_kernel_lse(dev):
    """Unit check of K2 alone: the oracle's backward given the kernel's own
    lse (the end-to-end checks above give it the oracle's)."""
    b = wl.logits_varlen(seed=2, device=dev)
    sl = slice(0, 128)
    _, lse = ilp.logp_selected(b.logits[sl], b.targets[sl], b.mask[sl])
    d = ilp.logp_backward(b.logits[sl], b.targets[sl], lse, b.grad[sl], b.mask[sl])
    torch.cuda.synchronize()
    rd = oracle.logp_backward(bits16(b.logits[sl]), b.targets[sl].cpu().numpy(),
                              b.mask[sl].cpu().numpy(), lse.cpu().numpy(), b.grad[sl].cpu().numpy())
    assert_close(d.cpu().numpy(), rd, TOL_BWD, "K2 given the kernel's lse")


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
