"""The C ABI's entry points allocate, free and synchronise nothing, so a caller
can capture them in a HIP graph.  One graph holds the logits path (forward
and backward), the fused path (forward, recomputing backward, kept-logits
forward and backward) and the parameter gradients; it is replayed several
times with the program's own eager work between replays, and every replay's
outputs equal the eager outputs bit for bit."""
import pytest
import torch

import invariant_logprob_amd as ilp
from gpu_util import f32bits, require_gpu
from invariant_logprob_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _run(c, f, out):
    """Every call writes into the preallocated buffers in `out`."""
    ilp.logp_selected(c.logits, c.targets, c.mask, logp=out["logp"], lse=out["lse"])
    ilp.logp_backward(c.logits, c.targets, out["lse"], c.grad, c.mask, out=out["d"])
    ilp.linear_logp(f.hidden, f.weight, f.targets, f.mask, workspace=out["ws"], logp=out["flogp"],
                    lse=out["flse"])
    ilp.linear_logp_backward(f.hidden, f.weight, f.targets, out["flse"], f.grad, f.mask,
                             out=out["fd"])
    ilp.linear_logp_with_logits(f.hidden, f.weight, f.targets, f.mask, workspace=out["ws"],
                                logp=out["klogp"], lse=out["klse"], logits=out["kz"])
    ilp.logp_backward(out["kz"], f.targets, out["klse"], f.grad, f.mask, out=out["kz"])
    ilp.linear_logp_param_grads(f.hidden, f.weight, f.targets, out["flse"], f.grad, f.mask,
                                grad_hidden=out["gh"], grad_weight=out["gw"], workspace=out["wsg"])


def _buffers(c, f, dev):
    n, v = c.logits.shape
    fn, h = f.hidden.shape
    fv = f.weight.shape[0]
    e = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
    return {"logp": e(n), "lse": e(n), "d": e(n, v), "flogp": e(fn), "flse": e(fn),
            "fd": e(fn, fv), "klogp": e(fn), "klse": e(fn), "kz": e(fn, fv), "gh": e(fn, h),
            "gw": e(fv, h),
            "ws": torch.empty(ilp.linear_logp_workspace_size(fn, fv, h), dtype=torch.uint8,
                              device=dev),
            "wsg": torch.empty(ilp.linear_logp_param_grads_workspace_size(fn, fv, h),
                               dtype=torch.uint8, device=dev)}


KEYS = ("logp", "lse", "d", "flogp", "flse", "fd", "klogp", "klse", "kz", "gh", "gw")


def test_graph_replays_match_eager():
    dev = require_gpu()
    ilp.load_library()
    c = wl.logits_batch(300, 5000, 3.0, seed=21, device=dev, n_masked=30)
    f = wl.fused_batch(200, 17000, 136, seed=22, device=dev, w_sigma=0.05, n_masked=15)
    eager = _buffers(c, f, dev)
    _run(c, f, eager)
    torch.cuda.synchronize()
    ref = {k: f32bits(eager[k]).clone() for k in KEYS}
    assert torch.equal(ref["kz"], ref["fd"])        # the kept-logits backward, in place

    out = _buffers(c, f, dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                   # warm up on the capture stream
        _run(c, f, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _run(c, f, out)
    for replay in range(3):
        for k in KEYS:                              # poison the outputs between replays
            out[k].fill_(float("nan"))
        scratch = torch.randn((1024, 1024), device=dev) @ torch.randn((1024, 1024), device=dev)
        g.replay()
        torch.cuda.synchronize()
        del scratch
        for k in KEYS:
            assert torch.equal(f32bits(out[k]), ref[k]), (replay, k)
