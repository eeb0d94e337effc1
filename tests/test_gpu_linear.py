"""GPU parity and bitwise invariance of the fused lm_head + selected logprob
(linear_logp, K3 + K4) and of its backward to the logits (K5), through the C
ABI, against the fp64 oracle.

Gradient references are end to end: the oracle's gradient from the bf16
hidden, weight, targets, mask and upstream gradient alone (its own lse).  One
separately named unit check feeds the kernel's lse to the oracle, to isolate
K5."""
import json
import math

import numpy as np
import pytest
import torch

import invariance as inv
import invariant_logprob_amd as ilp
import oracle
from gpu_util import TOL_BWD, TOL_FUSED, assert_close, bits16, f32bits, oracle_cached, require_gpu
from invariant_logprob_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    ilp.load_library()
    return d


def _oracle_fused(hidden, weight, targets, mask=None):
    return oracle.linear_logp(bits16(hidden), bits16(weight), targets.cpu().numpy(),
                              None if mask is None else mask.cpu().numpy())


@pytest.mark.parametrize("n,v,h", [(1, 256, 64), (37, 1000, 136), (300, 2600, 512), (257, 513, 8),
                                   (3, 1, 8), (40, 9, 16), (64, 257, 8)])
def test_small_parity_fwd_bwd(dev, n, v, h):
    b = wl.fused_batch(n, v, h, seed=n + v + h, device=dev, w_sigma=0.05, n_masked=n // 10)
    logp, lse = ilp.linear_logp(b.hidden, b.weight, b.targets, b.mask)
    torch.cuda.synchronize()
    rlogp, rlse = _oracle_fused(b.hidden, b.weight, b.targets, b.mask)
    act = b.mask.cpu().numpy().astype(bool)
    assert_close(logp.cpu().numpy(), rlogp, TOL_FUSED, f"fused logp {n}x{v}x{h}", act)
    assert_close(lse.cpu().numpy(), rlse, TOL_FUSED, f"fused lse {n}x{v}x{h}", act)
    assert bool((f32bits(logp)[~torch.from_numpy(act)] == 0).all())
    d = ilp.linear_logp_backward(b.hidden, b.weight, b.targets, lse, b.grad, b.mask)
    torch.cuda.synchronize()
    rd = oracle.linear_logp_backward(bits16(b.hidden), bits16(b.weight), b.targets.cpu().numpy(),
                                     b.mask.cpu().numpy(), rlse, b.grad.cpu().numpy())
    assert_close(d.cpu().numpy(), rd, TOL_BWD, f"fused dlogits {n}x{v}x{h} (end to end)")
    assert bool((f32bits(d)[~torch.from_numpy(act)] == 0).all())
    # unit check of K5 alone: the oracle's backward given the kernel's lse
    rd_k = oracle.linear_logp_backward(bits16(b.hidden), bits16(b.weight), b.targets.cpu().numpy(),
                                       b.mask.cpu().numpy(), lse.cpu().numpy(), b.grad.cpu().numpy())
    assert_close(d.cpu().numpy(), rd_k, TOL_BWD, f"K5 given the kernel's lse {n}x{v}x{h}")


def test_closed_forms(dev):
    v, h = 700, 128
    w = (torch.randn((v, h), device=dev) * 0.5).to(torch.bfloat16)
    hid = torch.zeros((5, h), dtype=torch.bfloat16, device=dev)   # z == 0 exactly
    t = torch.tensor([0, 1, 2, 3, 699], device=dev)
    logp, _ = ilp.linear_logp(hid, w, t)
    assert np.allclose(logp.cpu().numpy(), -math.log(v), atol=1e-5, rtol=0)
    # identical weight rows: uniform logits for any hidden row
    w2 = w[:1].repeat(v, 1).contiguous()
    hid2 = torch.randn((5, h), device=dev).to(torch.bfloat16)
    logp2, _ = ilp.linear_logp(hid2, w2, t)
    assert np.allclose(logp2.cpu().numpy(), -math.log(v), atol=1e-4, rtol=0)
    # invalid target on an active row -> NaN; masked row -> exactly 0
    t3 = torch.tensor([0, -1, 700, 5, 6], device=dev)
    mask = torch.tensor([1, 1, 1, 0, 1], dtype=torch.uint8, device=dev)
    logp3, lse3 = ilp.linear_logp(hid2, w, t3, mask)
    lp = logp3.cpu().numpy()
    assert np.isnan(lp[1]) and np.isnan(lp[2]) and not np.isnan(lp[0])
    assert int(f32bits(logp3)[3]) == 0
    d = ilp.linear_logp_backward(hid2, w, t3, lse3, torch.ones(5, device=dev), mask)
    assert bool(torch.isnan(d[1]).all()) and bool((f32bits(d[3]) == 0).all())


def _bits_equal(a, b):
    return torch.equal(f32bits(a), f32bits(b))


def test_tile_offset_sweep(dev):
    """The same token row at every kind of position inside a 256-row token
    block, among random neighbours, gives the bits it gives alone."""
    v, h = 1300, 256
    g = torch.Generator(device=dev).manual_seed(42)
    w = (torch.randn((v, h), generator=g, device=dev) * 0.05).to(torch.bfloat16)
    probe = torch.randn((3, h), generator=g, device=dev).to(torch.bfloat16)
    pt = torch.randint(0, v, (3,), generator=g, device=dev)
    alone = [ilp.linear_logp(probe[i:i + 1], w, pt[i:i + 1]) for i in range(3)]
    for off in (0, 1, 5, 31, 32, 33, 63, 64, 127, 128, 200, 255, 256, 300, 511):
        n = max(off + 1, 257) + 3
        hid = torch.randn((n, h), generator=g, device=dev).to(torch.bfloat16)
        tt = torch.randint(0, v, (n,), generator=g, device=dev)
        for i in range(3):
            hid[off] = probe[i]
            tt[off] = pt[i]
            lp, ls = ilp.linear_logp(hid, w, tt)
            assert int(f32bits(lp)[off]) == int(f32bits(alone[i][0])[0]), (off, i)
            assert int(f32bits(ls)[off]) == int(f32bits(alone[i][1])[0]), (off, i)


@pytest.mark.parametrize("v,h", [(1300, 136), (777, 72), (2600, 4096)])
def test_small_batch_forward_bits(dev, v, h):
    """Batches of at most 128 rows take the small-batch forward (register-staged
    W, 2, 4 or 8 waves per tile, 32, 64 or 128 token rows); each of their rows
    must carry the bits the same row gets inside a 300-row batch (the full
    tile forward), around every switch (N = 1, 2, 31, 32, 33, 63, 64, 65, 100,
    127, 128, 129), with a ragged last vocabulary tile and a ragged last K
    stage, a masked row and an invalid target among them; and the small
    batches agree with the oracle."""
    b = wl.fused_batch(300, v, h, seed=v + h, device=dev, w_sigma=0.05)
    t = b.targets.clone()
    t[2] = v + 5                      # invalid target on an active row
    m = b.mask.clone()
    m[4] = 0                          # masked row
    full_lp, full_ls = ilp.linear_logp(b.hidden, b.weight, t, m)
    for n in (1, 2, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129):
        lp, ls = ilp.linear_logp(b.hidden[:n], b.weight, t[:n], m[:n])
        assert torch.equal(f32bits(lp), f32bits(full_lp[:n])), n
        assert torch.equal(f32bits(ls), f32bits(full_ls[:n])), n
    lp, ls = ilp.linear_logp(b.hidden[:64], b.weight, t[:64], m[:64])
    keep = [r for r in range(64) if r not in (2, 4)]
    idx = torch.tensor(keep, device=dev)
    rlogp, rlse = _oracle_fused(b.hidden.index_select(0, idx), b.weight, t.index_select(0, idx))
    assert_close(lp.index_select(0, idx).cpu().numpy(), rlogp, TOL_FUSED, "small batch logp")
    assert_close(ls.index_select(0, idx).cpu().numpy(), rlse, TOL_FUSED, "small batch lse")
    assert math.isnan(float(lp[2])) and int(f32bits(lp[4:5])[0]) == 0


@pytest.mark.parametrize("v,h", [(1300, 136), (777, 72), (2600, 4096)])
def test_small_batch_backward_bits(dev, v, h):
    """Batches of at most 128 rows take the small-batch backward (the small
    forward's main loop, dlogits stored from the accumulators); each of their
    dlogits rows must carry the bits the same row gets inside a 300-row batch
    (the full tile backward), around both switches, with a ragged last
    vocabulary tile and a ragged last K stage, a masked row (all +0.0) and an
    invalid target on an active row (all NaN); and the 64-row batch agrees
    with the oracle's own gradient."""
    b = wl.fused_batch(300, v, h, seed=v + h + 1, device=dev, w_sigma=0.05)
    t = b.targets.clone()
    t[2] = v + 5                      # invalid target on an active row
    m = b.mask.clone()
    m[4] = 0                          # masked row
    _, full_ls = ilp.linear_logp(b.hidden, b.weight, t, m)
    full_d = ilp.linear_logp_backward(b.hidden, b.weight, t, full_ls, b.grad, m)
    for n in (1, 2, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129):
        d = ilp.linear_logp_backward(b.hidden[:n], b.weight, t[:n], full_ls[:n], b.grad[:n], m[:n])
        assert torch.equal(f32bits(d), f32bits(full_d[:n])), n
    d = ilp.linear_logp_backward(b.hidden[:64], b.weight, t[:64], full_ls[:64], b.grad[:64], m[:64])
    torch.cuda.synchronize()
    assert bool(torch.isnan(d[2]).all()) and bool((f32bits(d[4]) == 0).all())
    keep = [r for r in range(64) if r not in (2, 4)]
    idx = torch.tensor(keep, device=dev)
    sub_h, sub_t = b.hidden.index_select(0, idx), t.index_select(0, idx)
    _, rlse = _oracle_fused(sub_h, b.weight, sub_t)
    rd = oracle.linear_logp_backward(bits16(sub_h), bits16(b.weight), sub_t.cpu().numpy(), None,
                                     rlse, b.grad.index_select(0, idx).cpu().numpy())
    assert_close(d.index_select(0, idx).cpu().numpy(), rd, TOL_BWD,
                 f"small batch dlogits {v}x{h} (end to end)")


def test_fused_transforms_small(dev):
    n, v, h = 600, 1500, 192
    b = wl.fused_batch(n, v, h, seed=5, device=dev, w_sigma=0.05, n_masked=40)
    w = b.weight
    base = {"x": b.hidden, "targets": b.targets, "mask": b.mask, "grad": b.grad}

    def run(batch):
        logp, lse = ilp.linear_logp(batch["x"], w, batch["targets"], batch["mask"])
        d = ilp.linear_logp_backward(batch["x"], w, batch["targets"], lse, batch["grad"],
                                     batch["mask"])
        return {"logp": logp, "lse": lse, "dlogits": d}

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
        man = {"operator": "linear_logp", "chain_index": 7, "seed": 5,
               "transform": {"class": cls, "name": inv.TRANSFORM_NAMES[cls], **params}}
        recs, base_out = inv.check(run, base, calls, row_map, man, base_out)
        failures += recs
    assert not failures, json.dumps(failures[:3], indent=1)


def test_fused_large_config(dev):
    """hidden [8192, 4096], W [128256, 4096]: logp and lse of all 8192 rows
    against the oracle (about 8.6 TFLOP of fp64 products on the host, row
    blocks of 256 on all its cores: every MFMA column position of every token
    block, the ragged last vocabulary tile included); rows bitwise equal at
    N = 1, 33 and 8192."""
    b = wl.fused_large(seed=0, device=dev)
    logp, lse = ilp.linear_logp(b.hidden, b.weight, b.targets, b.mask)
    torch.cuda.synchronize()
    rlogp, rlse = _oracle_fused(b.hidden, b.weight, b.targets, b.mask)
    assert rlogp.shape == (8192,)
    assert_close(logp.cpu().numpy(), rlogp, TOL_FUSED, "C4 logp (all 8192 rows)")
    assert_close(lse.cpu().numpy(), rlse, TOL_FUSED, "C4 lse (all 8192 rows)")
    for r in (0, 1, 4095, 8191):
        one = ilp.linear_logp(b.hidden[r:r + 1], b.weight, b.targets[r:r + 1])
        assert _bits_equal(one[0], logp[r:r + 1]) and _bits_equal(one[1], lse[r:r + 1]), r
    s33 = ilp.linear_logp(b.hidden[4090:4123], b.weight, b.targets[4090:4123])
    assert _bits_equal(s33[0], logp[4090:4123]) and _bits_equal(s33[1], lse[4090:4123])


def c5_oracle_forward(b):
    """The oracle's (logp, lse) for every row of the hidden [2048, 5120],
    W [151936, 5120] workload (computed once per session)."""
    return oracle_cached(("fused_bwd", 0), lambda: _oracle_fused(b.hidden, b.weight, b.targets,
                                                                 b.mask))


def test_fused_backward_schedules(dev):
    """hidden [2048, 5120], W [151936, 5120]: logp and lse of all 2048 rows
    against the oracle; dlogits of 64 whole rows (both ends of each 512-row
    chunk among them) element by element against the oracle's own gradient;
    one prefill launch vs 4 chunks of 512 vs 2048 single-row decode launches
    give identical logp, lse and dlogits bits (dlogits of single rows and of
    32- and 64-row batches on a subset)."""
    b = wl.fused_bwd(seed=0, device=dev)
    n = b.hidden.shape[0]
    logp, lse = ilp.linear_logp(b.hidden, b.weight, b.targets, b.mask)
    d = ilp.linear_logp_backward(b.hidden, b.weight, b.targets, lse, b.grad, b.mask)
    torch.cuda.synchronize()
    rlogp, rlse = c5_oracle_forward(b)
    act = b.mask.cpu().numpy().astype(bool)
    assert act.all()
    assert_close(logp.cpu().numpy(), rlogp, TOL_FUSED, "C5 logp (all 2048 rows)")
    assert_close(lse.cpu().numpy(), rlse, TOL_FUSED, "C5 lse (all 2048 rows)")
    rows = sorted(set([0, 1, 511, 512, 1023, 1024, 1535, 1536, 2046, 2047] +
                      torch.randperm(n, generator=torch.Generator().manual_seed(6))[:80].tolist()))[:64]
    idx = torch.tensor(rows, device=dev)
    sub_h = b.hidden.index_select(0, idx)
    sub_t = b.targets.index_select(0, idx)
    rd = oracle.linear_logp_backward(bits16(sub_h), bits16(b.weight), sub_t.cpu().numpy(), None,
                                     rlse[rows], b.grad.index_select(0, idx).cpu().numpy())
    assert_close(d.index_select(0, idx).cpu().numpy(), rd, TOL_BWD,
                 "C5 dlogits (64 whole rows, end to end)")
    # 4 chunks of 512
    for c0 in range(0, n, 512):
        sl = slice(c0, c0 + 512)
        lp_c, ls_c = ilp.linear_logp(b.hidden[sl], b.weight, b.targets[sl], b.mask[sl])
        assert _bits_equal(lp_c, logp[sl]) and _bits_equal(ls_c, lse[sl]), c0
        d_c = ilp.linear_logp_backward(b.hidden[sl], b.weight, b.targets[sl], ls_c, b.grad[sl],
                                       b.mask[sl])
        assert _bits_equal(d_c, d[sl]), c0
    # one launch per row (decode); the dlogits rows are checked on a subset
    lp_rows = torch.empty_like(logp)
    ls_rows = torch.empty_like(lse)
    for r in range(n):
        ilp.linear_logp(b.hidden[r:r + 1], b.weight, b.targets[r:r + 1], b.mask[r:r + 1],
                        logp=lp_rows[r:r + 1], lse=ls_rows[r:r + 1])
    assert _bits_equal(lp_rows, logp) and _bits_equal(ls_rows, lse)
    for r in (0, 777, 2047):
        d_r = ilp.linear_logp_backward(b.hidden[r:r + 1], b.weight, b.targets[r:r + 1],
                                       lse[r:r + 1], b.grad[r:r + 1], b.mask[r:r + 1])
        assert _bits_equal(d_r, d[r:r + 1]), r
    # small batches (the small-batch backward) at this shape
    for r0, k in ((100, 32), (1000, 64), (1984, 64)):
        sl = slice(r0, r0 + k)
        d_k = ilp.linear_logp_backward(b.hidden[sl], b.weight, b.targets[sl], lse[sl], b.grad[sl],
                                       b.mask[sl])
        assert _bits_equal(d_k, d[sl]), (r0, k)


def test_binding_refuses_bad_outputs_and_workspaces(dev):
    """Caller-supplied outputs and workspaces are checked before any launch:
    a short output or a workspace that is too small, strided or on the host
    raises instead of letting a kernel write past it; an overlapping bf16
    backward output is refused by the library."""
    b = wl.fused_batch(40, 600, 64, seed=7, device=dev, w_sigma=0.05)
    need = ilp.linear_logp_workspace_size(40, 600, 64)
    short = torch.empty(39, dtype=torch.float32, device=dev)
    for kw in ({"logp": short}, {"lse": short}):
        with pytest.raises(ValueError):
            ilp.linear_logp(b.hidden, b.weight, b.targets, **kw)
        with pytest.raises(ValueError):
            ilp.linear_logp_with_logits(b.hidden, b.weight, b.targets, **kw)
    bad_ws = (torch.empty(need - 1, dtype=torch.uint8, device=dev),
              torch.empty(2 * need, dtype=torch.uint8, device=dev)[::2],
              torch.empty(need, dtype=torch.uint8))
    for ws in bad_ws:
        with pytest.raises(ValueError):
            ilp.linear_logp(b.hidden, b.weight, b.targets, workspace=ws)
        with pytest.raises(ValueError):
            ilp.linear_logp_param_grads(b.hidden, b.weight, b.targets, b.grad, b.grad,
                                        workspace=ws)
    # a good caller workspace gives the same bits as an internal one
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    a = ilp.linear_logp(b.hidden, b.weight, b.targets, workspace=ws)
    c = ilp.linear_logp(b.hidden, b.weight, b.targets)
    torch.cuda.synchronize()
    assert torch.equal(f32bits(a[0]), f32bits(c[0])) and torch.equal(f32bits(a[1]), f32bits(c[1]))
    # bf16 logits and an fp32 output that shares their memory
    buf = torch.zeros(8 * 1024, dtype=torch.float32, device=dev)
    x = buf.view(torch.bfloat16)[: 4 * 1024].view(4, 1024)
    t = torch.zeros(4, dtype=torch.int64, device=dev)
    lse = torch.zeros(4, dtype=torch.float32, device=dev)
    with pytest.raises(ilp.RlkError) as e:
        ilp.logp_backward(x, t, lse, lse, out=buf[: 4 * 1024].view(4, 1024))
    assert e.value.status == 1
    torch.cuda.synchronize()


def test_nonfinite_active_rows_reach_the_gradient(dev):
    """An active row whose hidden holds NaN (row 2) or +inf everywhere (row 5:
    with mixed-sign weight rows every logit is NaN) gets an all-NaN gradient
    row from the fused backward, from the backward over kept fp32 logits and
    from the parameter gradients (its grad_hidden row; grad_weight sums over
    it); on the bf16 logits path a row holding NaN or +inf likewise gets an
    all-NaN row.  Masked rows with the same poison give +0.0 everywhere, and
    the other rows keep the bits they have without the poisoned rows."""
    n, v, h = 12, 700, 64
    b = wl.fused_batch(n, v, h, seed=31, device=dev, w_sigma=0.05)
    hid = b.hidden.clone()
    hid[2, 7] = float("nan")
    hid[5, :] = float("inf")
    hid[8, ::2] = float("-inf")
    hid[9, 3] = float("nan")
    mask = torch.ones(n, dtype=torch.uint8, device=dev)
    mask[8] = 0
    mask[9] = 0
    w, t, g = b.weight, b.targets, b.grad
    _, lse = ilp.linear_logp(hid, w, t, mask)
    d = ilp.linear_logp_backward(hid, w, t, lse, g, mask)
    _, klse, z = ilp.linear_logp_with_logits(hid, w, t, mask)
    dk = ilp.logp_backward(z, t, klse, g, mask)
    gh, gw = ilp.linear_logp_param_grads(hid, w, t, lse, g, mask)
    torch.cuda.synchronize()
    clean_rows = [0, 1, 3, 4, 6, 7, 10, 11]
    ci = torch.tensor(clean_rows, device=dev)
    _, lse_c = ilp.linear_logp(hid[ci], w, t[ci])
    d_c = ilp.linear_logp_backward(hid[ci], w, t[ci], lse_c, g[ci])
    torch.cuda.synchronize()
    for name, dd in (("fused", d), ("kept logits", dk)):
        assert bool(torch.isnan(dd[2]).all()) and bool(torch.isnan(dd[5]).all()), name
        assert bool((f32bits(dd[8:10]) == 0).all()), name
        assert torch.equal(f32bits(dd[ci]), f32bits(d_c)), name
    assert bool(torch.isnan(gh[2]).all()) and bool(torch.isnan(gh[5]).all())
    assert bool((f32bits(gh[8:10]) == 0).all())
    assert bool(torch.isfinite(gh[ci]).all()) and bool(torch.isnan(gw).all())
    # bf16 logits path
    # (a width of 704: bf16 rows need a multiple of 8 elements; targets < 700)
    x = (torch.randn((n, 704), generator=torch.Generator(device=dev).manual_seed(3), device=dev)
         * 2).to(torch.bfloat16)
    x[2, 11] = float("nan")
    x[5, 40] = float("inf")
    x[6, ::5] = float("-inf")      # -inf entries only contribute zero
    x[8, 0] = float("nan")
    x[9, 1] = float("inf")
    _, lse_x = ilp.logp_selected(x, t, mask)
    dx = ilp.logp_backward(x, t, lse_x, g, mask)
    torch.cuda.synchronize()
    assert bool(torch.isnan(dx[2]).all()) and bool(torch.isnan(dx[5]).all())
    assert bool(torch.isfinite(dx[6]).all())
    assert bool((f32bits(dx[8:10]) == 0).all())
