"""GPU parity and invariance of the fused path's parameter gradients,
grad_hidden = D . W and grad_weight = D^T . h (D the logits gradient),
through the C ABI, against the fp64 oracle.

Tolerance, fixed before any measurement and independent of how the library
forms its operands: the target's backward bound |delta| <= 1e-3 for every
gradient entry, and an fp32-grade bound |delta| <= 1e-4 S + 1e-5, where S is
the sum of the absolute values of the summed terms (sum_j |D_ij| |W_jk| for
grad_hidden[i, k], sum_i |D_ij| |h_ik| for grad_weight[j, k]); see
gpu_util.param_tol.  References are end to end: the oracle's gradients from
the bf16 inputs, targets, mask and upstream gradient alone, with its own
log-sum-exp.
"""
import json

import numpy as np
import pytest
import torch

import invariance as inv
import invariant_logprob_amd as ilp
import oracle
from gpu_util import assert_close, bits16, f32bits, oracle_cached, param_tol, require_gpu
from invariant_logprob_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    ilp.load_library()
    return d


def _bits_equal(a, b):
    return torch.equal(f32bits(a), f32bits(b))


def _grads(b, lse, **kw):
    gh, gw = ilp.linear_logp_param_grads(b.hidden, b.weight, b.targets, lse, b.grad, b.mask, **kw)
    torch.cuda.synchronize()
    return gh, gw


@pytest.mark.parametrize("n,v,h", [(1, 256, 64), (33, 1000, 256), (300, 17000, 136),
                                   (257, 513, 8)])
def test_small_parity(dev, n, v, h):
    """Several tiles, a ragged token block, a ragged vocabulary chunk (17000
    = one full 16384 chunk + a partial one) and a ragged K (H = 136)."""
    b = wl.fused_batch(n, v, h, seed=n + v + h + 1, device=dev, w_sigma=0.05, n_masked=n // 10)
    _, lse = ilp.linear_logp(b.hidden, b.weight, b.targets, b.mask)
    gh, gw = _grads(b, lse)
    hb, wb = bits16(b.hidden), bits16(b.weight)
    t = b.targets.cpu().numpy()
    m = b.mask.cpu().numpy()
    g = b.grad.cpu().numpy()
    # end to end: lse=None makes the oracle take its own log-sum-exp
    rgh, rgw = oracle.linear_param_grads(hb, wb, t, m, None, g)
    d_abs = np.abs(oracle.linear_logp_backward(hb, wb, t, m, None, g))
    h_abs = np.abs(oracle.bf16_to_f64(hb))
    w_abs = np.abs(oracle.bf16_to_f64(wb))
    assert_close(gh.cpu().numpy(), rgh, param_tol(d_abs @ w_abs), f"grad_hidden {n}x{v}x{h}")
    assert_close(gw.cpu().numpy(), rgw, param_tol(d_abs.T @ h_abs), f"grad_weight {n}x{v}x{h}")
    inactive = torch.from_numpy(m == 0)
    assert bool((f32bits(gh)[inactive] == 0).all()), "inactive rows must be +0.0"
    # one output at a time gives the same bits
    gh1, none1 = _grads(b, lse, want_weight=False)
    none2, gw2 = _grads(b, lse, want_hidden=False)
    assert none1 is None and none2 is None
    assert _bits_equal(gh1, gh) and _bits_equal(gw2, gw)


def test_closed_forms(dev):
    v, h = 600, 64
    w = (torch.randn((v, h), device=dev) * 0.5).to(torch.bfloat16)
    # zero hidden rows: logits 0, p = 1/V, grad_h_i = g_i (W[t_i] - mean_j W_j), grad_W = 0
    hid = torch.zeros((4, h), dtype=torch.bfloat16, device=dev)
    t = torch.tensor([0, 17, 300, 599], device=dev)
    g = torch.tensor([1.0, -2.0, 0.5, 0.0], device=dev)
    _, lse = ilp.linear_logp(hid, w, t)
    gh, gw = ilp.linear_logp_param_grads(hid, w, t, lse, g)
    torch.cuda.synchronize()
    w64 = w.double().cpu()
    ref = g.double().cpu()[:, None] * (w64[t.cpu()] - w64.mean(dim=0))
    # sum_j |D_ij| |W_jk| = |g_i| (|W_t,k| (1 - 1/V) + mean_j |W_jk| - |W_t,k| / V)
    scale = (g.double().abs().cpu()[:, None] * (w64[t.cpu()].abs() + w64.abs().mean(dim=0)))
    assert_close(gh.cpu().numpy(), ref.numpy(), param_tol(scale.numpy()), "zero-hidden grad_h")
    assert float(gw.abs().max()) == 0.0
    # a row with g = 0 has zero hidden gradient bits
    assert bool((f32bits(gh[3]) == 0).all())


def test_invalid_target_and_empty_batch(dev):
    v, h = 300, 64
    b = wl.fused_batch(5, v, h, seed=3, device=dev, w_sigma=0.05)
    t = b.targets.clone()
    t[2] = v        # active row with an invalid target
    _, lse = ilp.linear_logp(b.hidden, b.weight, t)
    gh, gw = ilp.linear_logp_param_grads(b.hidden, b.weight, t, lse, b.grad)
    torch.cuda.synchronize()
    assert bool(torch.isnan(gh[2]).all())
    assert bool(torch.isfinite(gh[[0, 1, 3, 4]]).all())
    assert bool(torch.isnan(gw).all()), "an invalid active target must poison grad_weight"
    # N == 0: grad_weight is the empty sum, written as zeros
    gw0 = torch.full((v, h), float("nan"), device=dev)
    e = torch.empty((0, h), dtype=torch.bfloat16, device=dev)
    z = torch.empty((0,), device=dev)
    ilp.linear_logp_param_grads(e, b.weight, torch.empty((0,), dtype=torch.int64, device=dev), z, z,
                                want_hidden=False, grad_weight=gw0)
    torch.cuda.synchronize()
    assert bool((f32bits(gw0) == 0).all())


def test_grad_hidden_transforms(dev):
    """grad_hidden rows are bitwise invariant under T1-T6 (the harness
    compares raw bits of every active row)."""
    n, v, h = 520, 17000, 128
    b = wl.fused_batch(n, v, h, seed=9, device=dev, w_sigma=0.05, n_masked=30)
    w = b.weight
    base = {"x": b.hidden, "targets": b.targets, "mask": b.mask, "grad": b.grad}

    def run(batch):
        _, lse = ilp.linear_logp(batch["x"], w, batch["targets"], batch["mask"])
        gh, _ = ilp.linear_logp_param_grads(batch["x"], w, batch["targets"], lse, batch["grad"],
                                            batch["mask"], want_weight=False)
        return {"lse": lse, "grad_hidden": gh}

    def filler(k, seed):
        gg = torch.Generator(device=dev).manual_seed(seed)
        return {"x": (torch.randn((k, h), generator=gg, device=dev) * 3).to(torch.bfloat16),
                "targets": torch.randint(0, v, (k,), generator=gg, device=dev),
                "mask": torch.ones(k, dtype=torch.uint8, device=dev),
                "grad": torch.randn((k,), generator=gg, device=dev)}

    cases = [("T1", {"size": s, "start": st}, inv.t1_population(base, s, st))
             for s, st in ((1, 0), (33, 5), (257, 100))]
    cases += [("T2", {"seed": 1}, inv.t2_position(base, 1)),
              ("T3", {"keep": "every 7th"}, inv.t3_neighbours(base, list(range(0, n, 7)), filler, 2)),
              ("T4", {"left": 9, "every": 50}, inv.t4_padding(base, filler, 3, left=9, right=4, every=50)),
              ("T5", {"chunk": 128}, inv.t5_schedule(base, 128)),
              ("T6", {"compacted": True}, inv.t6_compacted(base))]
    failures = []
    base_out = None
    for cls, params, (calls, row_map) in cases:
        man = {"operator": "linear_logp.grad_hidden", "chain_index": 7, "seed": 9,
               "transform": {"class": cls, "name": inv.TRANSFORM_NAMES[cls], **params}}
        recs, base_out = inv.check(run, base, calls, row_map, man, base_out)
        failures += recs
    assert not failures, json.dumps(failures[:3], indent=1)


def test_grad_weight_determinism_and_layouts(dev):
    """grad_weight sums over the whole batch: bitwise run to run and under
    masked rows appended after the batch; a permuted batch is another sum
    order, equal within the derived tolerance."""
    n, v, h = 400, 3000, 192
    b = wl.fused_batch(n, v, h, seed=21, device=dev, w_sigma=0.05, n_masked=20)
    _, lse = ilp.linear_logp(b.hidden, b.weight, b.targets, b.mask)
    _, gw = _grads(b, lse, want_hidden=False)
    _, gw_again = _grads(b, lse, want_hidden=False)
    assert _bits_equal(gw, gw_again)
    # 77 masked rows with random content and invalid targets after the batch
    k = 77
    gg = torch.Generator(device=dev).manual_seed(5)
    hid2 = torch.cat([b.hidden, (torch.randn((k, h), generator=gg, device=dev) * 3).to(torch.bfloat16)])
    t2 = torch.cat([b.targets, torch.full((k,), -100, dtype=torch.int64, device=dev)])
    m2 = torch.cat([b.mask, torch.zeros(k, dtype=torch.uint8, device=dev)])
    g2 = torch.cat([b.grad, torch.randn((k,), generator=gg, device=dev)])
    lse2 = torch.cat([lse, torch.zeros(k, device=dev)])
    _, gw_pad = ilp.linear_logp_param_grads(hid2, b.weight, t2, lse2, g2, m2, want_hidden=False)
    torch.cuda.synchronize()
    assert _bits_equal(gw_pad, gw)
    # permutation: same set of samples, another order of the sum
    perm = torch.randperm(n, generator=gg, device=dev)
    _, gw_perm = ilp.linear_logp_param_grads(b.hidden[perm], b.weight, b.targets[perm], lse[perm],
                                             b.grad[perm], b.mask[perm], want_hidden=False)
    torch.cuda.synchronize()
    hb, wb = bits16(b.hidden), bits16(b.weight)
    d_abs = np.abs(oracle.linear_logp_backward(hb, wb, b.targets.cpu().numpy(), b.mask.cpu().numpy(),
                                               None, b.grad.cpu().numpy()))
    scale = d_abs.T @ np.abs(oracle.bf16_to_f64(hb))
    # two sums of the same terms, each within param_tol of the exact value
    assert_close(gw_perm.cpu().numpy(), gw.cpu().numpy().astype(np.float64), 2 * param_tol(scale),
                 "grad_weight under a permutation")


def test_full_size_sampled(dev):
    """hidden [2048, 5120], W [151936, 5120]: sampled rows of both gradients
    against the oracle's end-to-end gradients (its lse from its own forward
    over all 2048 rows); grad_hidden rows bitwise equal from a 512-row call
    and from single-row calls."""
    b = wl.fused_bwd(seed=0, device=dev)
    n = b.hidden.shape[0]
    _, lse = ilp.linear_logp(b.hidden, b.weight, b.targets, b.mask)
    gh, gw = _grads(b, lse)
    hb, wb = bits16(b.hidden), bits16(b.weight)
    t = b.targets.cpu().numpy()
    m = b.mask.cpu().numpy()
    g = b.grad.cpu().numpy()
    _, ls = oracle_cached(("fused_bwd", 0), lambda: oracle.linear_logp(hb, wb, t, m))
    rows = [0, 777, 2047]
    rgh = oracle.linear_grad_hidden_rows(hb, wb, t, m, ls, g, rows)
    w64 = oracle.bf16_to_f64(wb)
    d_rows = oracle.logp_backward_from_f64(oracle.bf16_to_f64(hb[rows]) @ w64.T, t[rows], m[rows],
                                           ls[rows], g[rows])
    bound_h = np.abs(d_rows) @ np.abs(w64)
    del w64
    assert_close(gh[rows].cpu().numpy(), rgh, param_tol(bound_h), "C5 grad_hidden rows")
    vrows = sorted({int(t[0]), int(t[1000]), 0, 75000, 151935})
    rgw = oracle.linear_grad_weight_rows(hb, wb, t, m, ls, g, vrows)
    h64 = oracle.bf16_to_f64(hb)
    z = h64 @ oracle.bf16_to_f64(wb[vrows]).T
    act = m.astype(bool)
    p = np.exp(z - ls[:, None])
    onehot = (t[:, None] == np.asarray(vrows)[None, :]).astype(np.float64)
    d_cols = np.where(act[:, None], g[:, None] * (onehot - p), 0.0)
    bound_w = np.abs(d_cols).T @ np.abs(h64)
    assert_close(gw[vrows].cpu().numpy(), rgw, param_tol(bound_w), "C5 grad_weight rows")
    sl = slice(512, 1024)
    gh_c, _ = ilp.linear_logp_param_grads(b.hidden[sl], b.weight, b.targets[sl], lse[sl], b.grad[sl],
                                          b.mask[sl], want_weight=False)
    torch.cuda.synchronize()
    assert _bits_equal(gh_c, gh[sl])
    for r in (0, 777, n - 1):
        gh_r, _ = ilp.linear_logp_param_grads(b.hidden[r:r + 1], b.weight, b.targets[r:r + 1],
                                              lse[r:r + 1], b.grad[r:r + 1], b.mask[r:r + 1],
                                              want_weight=False)
        torch.cuda.synchronize()
        assert _bits_equal(gh_r, gh[r:r + 1]), r


def test_autograd_wrapper(dev):
    n, v, h = 70, 900, 64
    b = wl.fused_batch(n, v, h, seed=4, device=dev, w_sigma=0.05, n_masked=5)
    hid = b.hidden.clone().requires_grad_(True)
    w = b.weight.clone().requires_grad_(True)
    logp = ilp.LinearLogprob.apply(hid, w, b.targets, b.mask)
    (logp * b.grad).sum().backward()
    _, lse = ilp.linear_logp(b.hidden, b.weight, b.targets, b.mask)
    gh, gw = _grads(b, lse)
    assert hid.grad.dtype == torch.bfloat16 and w.grad.dtype == torch.bfloat16
    assert torch.equal(hid.grad, gh.to(torch.bfloat16))
    assert torch.equal(w.grad, gw.to(torch.bfloat16))
    # keeping the logits for the backward gives the same gradients
    hid2 = b.hidden.clone().requires_grad_(True)
    w2 = b.weight.clone().requires_grad_(True)
    logp2 = ilp.LinearLogprob.apply(hid2, w2, b.targets, b.mask, True)
    (logp2 * b.grad).sum().backward()
    assert torch.equal(logp2.detach().view(torch.int32), logp.detach().view(torch.int32))
    assert torch.equal(hid2.grad, hid.grad) and torch.equal(w2.grad, w.grad)


def test_padded_leading_dimensions(dev):
    """hidden and weight as views of wider buffers (ld = H + 24, + 8), and
    outputs with ld = H + 12: the K-major operand reads follow the leading
    dimensions, and the results equal those of contiguous copies bit for bit."""
    n, v, h = 150, 1700, 200
    b = wl.fused_batch(n, v, h, seed=17, device=dev, w_sigma=0.05, n_masked=11)
    hb = torch.full((n, h + 24), float("nan"), device=dev).to(torch.bfloat16)
    hb[:, :h] = b.hidden
    wb = torch.full((v, h + 8), float("nan"), device=dev).to(torch.bfloat16)
    wb[:, :h] = b.weight
    hid, wei = hb[:, :h], wb[:, :h]
    logp, lse = ilp.linear_logp(b.hidden, b.weight, b.targets, b.mask)
    gh, gw = _grads(b, lse)
    # the forward and the logits backward on the padded views give the same bits
    logp2, lse2 = ilp.linear_logp(hid, wei, b.targets, b.mask)
    d = ilp.linear_logp_backward(b.hidden, b.weight, b.targets, lse, b.grad, b.mask)
    d2 = ilp.linear_logp_backward(hid, wei, b.targets, lse, b.grad, b.mask)
    torch.cuda.synchronize()
    assert _bits_equal(logp2, logp) and _bits_equal(lse2, lse) and _bits_equal(d2, d)
    gh_buf = torch.full((n, h + 12), float("nan"), device=dev)
    gw_buf = torch.full((v, h + 12), float("nan"), device=dev)
    gh2, gw2 = ilp.linear_logp_param_grads(hid, wei, b.targets, lse, b.grad, b.mask,
                                           grad_hidden=gh_buf[:, :h], grad_weight=gw_buf[:, :h])
    torch.cuda.synchronize()
    assert _bits_equal(gh2, gh) and _bits_equal(gw2, gw)
    # columns past H of the output buffers are never written
    assert bool(torch.isnan(gh_buf[:, h:]).all()) and bool(torch.isnan(gw_buf[:, h:]).all())


def test_inactive_rows_may_hold_anything(dev):
    """Inactive tokens add nothing, whatever their hidden rows hold: with NaN
    and infinities in masked rows (padding is often uninitialised memory),
    both gradients, the forward and the logits backward equal, bit for bit,
    those of the same batch with those rows zeroed."""
    n, v, h = 300, 17000, 136
    b = wl.fused_batch(n, v, h, seed=77, device=dev, w_sigma=0.05, n_masked=30)
    masked = torch.nonzero(b.mask == 0).flatten()[:3]
    poisoned = b.hidden.clone()
    poisoned[masked[0], 5] = float("nan")
    poisoned[masked[1], :] = float("inf")
    poisoned[masked[2], ::3] = float("-inf")
    clean = b.hidden.clone()
    clean[masked] = 0
    outs = []
    for hid in (poisoned, clean):
        logp, lse = ilp.linear_logp(hid, b.weight, b.targets, b.mask)
        d = ilp.linear_logp_backward(hid, b.weight, b.targets, lse, b.grad, b.mask)
        gh, gw = ilp.linear_logp_param_grads(hid, b.weight, b.targets, lse, b.grad, b.mask)
        _, _, z = ilp.linear_logp_with_logits(hid, b.weight, b.targets, b.mask)
        gh2, gw2 = ilp.linear_logp_param_grads(hid, b.weight, b.targets, lse, b.grad, b.mask,
                                               logits=z)
        torch.cuda.synchronize()
        outs.append([logp, lse, d, gh, gw, gh2, gw2])
    assert bool(torch.isfinite(outs[0][4]).all()), "grad_weight took in an inactive row"
    for name, a, c in zip(("logp", "lse", "dlogits", "grad_hidden", "grad_weight",
                           "grad_hidden (kept)", "grad_weight (kept)"), outs[0], outs[1]):
        assert _bits_equal(a, c), name
