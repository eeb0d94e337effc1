"""GPU parity and invariance of the dense-path outputs: per-row entropy
(rlk_logp_entropy) and dense log-softmax rows (rlk_log_softmax), against
the fp64 oracle, through the C ABI.

Tolerances.  Dense log-softmax entries are one fp32 subtraction away from
the logits-path lse, so they take the logits-path bound
|d| <= 2e-5 + 1e-5 |r|.  The entropy adds a second fp32 sum (sum_j p_j x_j,
weights up to E_p|x| ~ 20 at these widths) whose accumulated rounding can
reach a few 1e-5, so its bound is |d| <= 1e-4 + 1e-5 |r|."""
import json
import math

import numpy as np
import pytest
import torch

import invariance as inv
import invariant_logprob_amd as ilp
import oracle
from gpu_util import assert_close, bits16, f32bits, padded_bf16, require_gpu, tol_logits
from invariant_logprob_amd import workloads as wl

pytestmark = pytest.mark.gpu


def tol_entropy(r):
    return 1e-4 + 1e-5 * np.abs(r)


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    ilp.load_library()
    return d


def _check(logits, targets, mask, what):
    logp, lse, ent = ilp.logp_entropy(logits, targets, mask)
    lp2, lse2 = ilp.logp_selected(logits, targets, mask)
    torch.cuda.synchronize()
    # the entropy kernel's logp / lse are the plain kernel's, bit for bit
    assert torch.equal(f32bits(logp), f32bits(lp2)) and torch.equal(f32bits(lse), f32bits(lse2))
    bits = bits16(logits)
    m = None if mask is None else mask.cpu().numpy()
    act = np.ones(bits.shape[0], bool) if m is None else m.astype(bool)
    ref = oracle.entropy(bits, m)
    assert_close(ent.cpu().numpy(), ref, tol_entropy, f"{what} entropy", act)
    assert bool((f32bits(ent)[~torch.from_numpy(act)] == 0).all())
    return lse


@pytest.mark.parametrize("v", [1, 3, 8, 1024, 2049, 32000])
def test_entropy_parity(dev, v):
    n = 9
    g = torch.Generator(device=dev).manual_seed(100 + v)
    x = (torch.randn((n, v), generator=g, device=dev) * 3).to(torch.bfloat16)
    logits = padded_bf16(n, v, (v + 7) // 8 * 8, x)
    t = torch.randint(0, v, (n,), generator=g, device=dev)
    mask = torch.tensor([1, 1, 0, 1, 1, 1, 1, 0, 1], dtype=torch.uint8, device=dev)
    _check(logits, t, mask, f"V={v}")


def test_entropy_closed_forms(dev):
    for v in (1, 1000, 151936):
        ld = (v + 7) // 8 * 8
        x = padded_bf16(2, v, ld, torch.full((2, v), -1.5, dtype=torch.bfloat16, device=dev))
        _, _, ent = ilp.logp_entropy(x, torch.zeros(2, dtype=torch.int64, device=dev))
        assert np.allclose(ent.cpu().numpy(), math.log(v), atol=1e-4 + 1e-5 * math.log(v), rtol=0)
    # -inf entries contribute nothing
    v = 4000
    x = torch.zeros((1, v), device=dev)
    x[0, 1::2] = float("-inf")
    _, _, ent = ilp.logp_entropy(x.to(torch.bfloat16), torch.zeros(1, dtype=torch.int64, device=dev))
    assert abs(float(ent[0]) - math.log(v // 2)) <= 1e-4


def test_entropy_large_sampled(dev):
    b = wl.logits_large(seed=0, device=dev)
    logp, lse, ent = ilp.logp_entropy(b.logits, b.targets, b.mask)
    lp2, _ = ilp.logp_selected(b.logits, b.targets, b.mask)
    torch.cuda.synchronize()
    assert torch.equal(f32bits(logp), f32bits(lp2))
    rows = torch.randperm(b.logits.shape[0], generator=torch.Generator().manual_seed(9))[:32]
    idx = rows.to(dev)
    m = b.mask.index_select(0, idx).cpu().numpy()
    ref = oracle.entropy(bits16(b.logits.index_select(0, idx)), m)
    assert_close(ent.index_select(0, idx).cpu().numpy(), ref, tol_entropy, "large entropy",
                 m.astype(bool))


def test_entropy_invariance(dev):
    v, n = 151936, 300
    b = wl.logits_batch(n, v, 4.0, seed=3, device=dev, n_masked=30)
    base = {"x": b.logits, "targets": b.targets, "mask": b.mask}

    def run(batch):
        lp, lse, ent = ilp.logp_entropy(batch["x"], batch["targets"], batch["mask"])
        return {"logp": lp, "lse": lse, "entropy": ent}

    def filler(k, seed):
        x, t = wl.neighbour_rows(k, v, seed, device=dev)
        return {"x": x, "targets": t, "mask": torch.ones(k, dtype=torch.uint8, device=dev)}

    cases = [("T1", {"size": 1}, inv.t1_population(base, 1, 17)),
             ("T1", {"size": 7}, inv.t1_population(base, 7, 100)),
             ("T2", {"seed": 5}, inv.t2_position(base, 5)),
             ("T3", {"keep": "every 11th"}, inv.t3_neighbours(base, list(range(0, n, 11)), filler, 6)),
             ("T4", {"every": 50}, inv.t4_padding(base, filler, 7, left=2, right=3, every=50)),
             ("T5", {"chunk": 1}, inv.t5_schedule(base, 1)),
             ("T6", {"compacted": True}, inv.t6_compacted(base))]
    fails = []
    base_out = None
    for cls, params, (calls, row_map) in cases:
        man = {"operator": "logp_entropy", "chain_index": 8, "seed": 3,
               "transform": {"class": cls, "name": inv.TRANSFORM_NAMES[cls], **params}}
        recs, base_out = inv.check(run, base, calls, row_map, man, base_out)
        fails += recs
    assert not fails, json.dumps(fails[:3], indent=1)


def test_log_softmax_parity_and_invariance(dev):
    for v in (5, 2049, 32000):
        n = 7
        g = torch.Generator(device=dev).manual_seed(200 + v)
        x = (torch.randn((n, v), generator=g, device=dev) * 3).to(torch.bfloat16)
        logits = padded_bf16(n, v, (v + 7) // 8 * 8, x)
        t = torch.randint(0, v, (n,), generator=g, device=dev)
        mask = torch.tensor([1, 0, 1, 1, 1, 1, 1], dtype=torch.uint8, device=dev)
        _, lse = ilp.logp_selected(logits, t, mask)
        ls = ilp.log_softmax(logits, lse, mask)
        torch.cuda.synchronize()
        ref = oracle.log_softmax(bits16(logits), mask.cpu().numpy())
        assert_close(ls.cpu().numpy(), ref, tol_logits, f"log_softmax V={v}")
        assert bool((f32bits(ls[1]) == 0).all())
        # its selected entries are the selected logprobs' values (same lse)
        sel = ls.gather(1, t.clamp(min=0).view(-1, 1)).flatten()
        lp, _ = ilp.logp_selected(logits, t, mask)
        act = mask.bool()
        assert torch.equal(f32bits(sel[act]), f32bits(lp[act]))
    # invariance: a row alone vs inside a batch
    b = wl.logits_varlen(seed=2, device=dev)
    _, lse = ilp.logp_selected(b.logits, b.targets, b.mask)
    full = ilp.log_softmax(b.logits, lse, b.mask)
    for r in (0, 500, 1777):
        one = ilp.log_softmax(b.logits[r:r + 1], lse[r:r + 1], b.mask[r:r + 1])
        assert torch.equal(f32bits(one), f32bits(full[r:r + 1]))
