"""Bitwise batch invariance (relation I) of the logits path on the GPU under
the transform classes T1-T6 (page "docs(ws1): batch-invariance contract RFC",
PR summary and section "T5: Execution schedule"; page "[RFC] Batch-Invariant
RL Kernel Suite for Train-Inference Consistency", maintainer reply: bitwise,
atol = rtol = 0).  Forward (logp, lse) and backward (dlogits rows) are
compared as raw 32-bit patterns."""
import json

import pytest
import torch

import invariance as inv
import invariant_logprob_amd as ilp
from gpu_util import require_gpu
from invariant_logprob_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    ilp.load_library()
    return d


def run_fwd(batch):
    logp, lse = ilp.logp_selected(batch["x"], batch["targets"], batch["mask"])
    return {"logp": logp, "lse": lse}


def run_fwd_bwd(batch):
    logp, lse = ilp.logp_selected(batch["x"], batch["targets"], batch["mask"])
    d = ilp.logp_backward(batch["x"], batch["targets"], lse, batch["grad"], batch["mask"])
    return {"logp": logp, "lse": lse, "dlogits": d}


def filler_for(v, dev, with_grad=False):
    def f(n, seed):
        x, t = wl.neighbour_rows(n, v, seed, device=dev)
        rows = {"x": x, "targets": t, "mask": torch.ones(n, dtype=torch.uint8, device=dev)}
        if with_grad:
            rows["grad"] = torch.randn((n,), generator=torch.Generator(device=dev).manual_seed(seed),
                                       device=dev)
        return rows
    return f


def _assert_invariant(run, base, cases, op="logp", base_out=None):
    failures = []
    for cls, params, (calls, row_map) in cases:
        man = {"operator": op, "chain_index": 8, "seed": 0, "device": "cuda:0",
               "transform": {"class": cls, "name": inv.TRANSFORM_NAMES[cls], **params},
               "launch": {"rows": [inv.nrows(c) for c in calls][:4], "calls": len(calls)}}
        recs, base_out = inv.check(run, base, calls, row_map, man, base_out)
        failures += recs
    assert not failures, json.dumps(failures[:3], indent=1)


def test_small_config_b1_vs_b8_permuted(dev):
    b = wl.logits_small(seed=0, device=dev)
    base = {"x": b.logits, "targets": b.targets, "mask": b.mask, "grad": b.grad}
    perm_calls, perm_map = inv.t2_position(base, 0)
    cases = [("T2", {"perm_seed": 0}, (perm_calls, perm_map))]
    cases += [("T1", {"size": 1, "start": s}, inv.t1_population(base, 1, start=s)) for s in range(8)]
    _assert_invariant(run_fwd_bwd, base, cases)


def test_large_vocab_transforms(dev):
    """V=151936 with batch sizes {1, 7, 64, 257, 1024}, shuffles, fresh
    neighbours, padding and split launches."""
    v, n = 151936, 1024
    b = wl.logits_batch(n, v, 4.0, seed=0, device=dev, n_masked=int(round(0.15 * n)))
    base = {"x": b.logits, "targets": b.targets, "mask": b.mask}
    filler = filler_for(v, dev)
    cases = []
    for size in (1, 7, 64, 257):
        for start in (0, 300, 1000):
            cases.append(("T1", {"size": size, "start": start}, inv.t1_population(base, size, start)))
    for seed in (1, 2):
        cases.append(("T2", {"seed": seed}, inv.t2_position(base, seed)))
    keep = list(range(0, n, 37))
    cases.append(("T3", {"keep": "every 37th", "seed": 3}, inv.t3_neighbours(base, keep, filler, 3)))
    cases.append(("T4", {"left": 5, "right": 11, "every": 100},
                  inv.t4_padding(base, filler, 4, left=5, right=11, every=100)))
    cases.append(("T5", {"chunk": 100}, inv.t5_schedule(base, 100)))
    cases.append(("T6", {"compacted": True}, inv.t6_compacted(base)))
    _assert_invariant(run_fwd, base, cases)


def test_large_vocab_decode_schedule(dev):
    """T5: one prefill launch vs one launch per row (decode)."""
    v, n = 151936, 96
    b = wl.logits_batch(n, v, 4.0, seed=7, device=dev)
    base = {"x": b.logits, "targets": b.targets, "mask": b.mask, "grad": b.grad}
    _assert_invariant(run_fwd_bwd, base, [("T5", {"chunk": 1}, inv.t5_schedule(base, 1)),
                                          ("T5", {"chunk": 32}, inv.t5_schedule(base, 32))])


def test_varlen_packing_layouts(dev):
    """T6: packed varlen rows vs right- and left-padded [B, S_max] layouts;
    T4: padding rows interleaved; backward rows included."""
    b = wl.logits_varlen(seed=0, device=dev)
    total = sum(b.seq_lens)
    base = {"x": b.logits[:total], "targets": b.targets[:total], "mask": b.mask[:total],
            "grad": b.grad[:total]}
    filler = filler_for(b.logits.shape[1], dev, with_grad=True)
    s_max = max(b.seq_lens)
    cases = [
        ("T6", {"padded": "right", "s_max": s_max},
         inv.t6_padded_layout(base, b.seq_lens, s_max, filler, 11, "right")),
        ("T6", {"padded": "left", "s_max": s_max},
         inv.t6_padded_layout(base, b.seq_lens, s_max, filler, 12, "left")),
        ("T4", {"every": 64}, inv.t4_padding(base, filler, 13, left=3, right=2, every=64)),
    ]

    def run(batch):
        out = run_fwd(batch)
        return out
    _assert_invariant(run, base, cases)
    # backward on the first sequence only (dense [rows, V] outputs)
    L0 = b.seq_lens[0]
    sub = {k: v[:L0] for k, v in base.items()}
    cases_b = [("T1", {"size": 17, "start": 3}, inv.t1_population(sub, 17, 3)),
               ("T2", {"seed": 4}, inv.t2_position(sub, 4)),
               ("T5", {"chunk": 1}, inv.t5_schedule(sub, 1))]
    _assert_invariant(run_fwd_bwd, sub, cases_b)


def test_strided_rows_match_contiguous(dev):
    """The same row read from a wider buffer (a different leading dimension)
    gives the same bits: the lane map depends on the column only."""
    v, n = 32000, 16
    b = wl.logits_batch(n, v, 3.0, seed=9, device=dev)
    wide = torch.empty((n, v + 64), dtype=torch.bfloat16, device=dev)
    wide[:, v:] = float("nan")
    wide[:, :v] = b.logits
    a = ilp.logp_selected(b.logits, b.targets)
    c = ilp.logp_selected(wide[:, :v], b.targets)
    assert torch.equal(a[0].view(torch.int32), c[0].view(torch.int32))
    assert torch.equal(a[1].view(torch.int32), c[1].view(torch.int32))
