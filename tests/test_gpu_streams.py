"""The library keeps no state between calls, so calls on different streams,
and from several host threads at once, give the same bits as the same calls
made one after another on one stream."""
import threading

import pytest
import torch

import invariant_logprob_amd as ilp
from gpu_util import f32bits, require_gpu
from invariant_logprob_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    ilp.load_library()
    return d


def _fused(f):
    logp, lse = ilp.linear_logp(f.hidden, f.weight, f.targets, f.mask)
    d = ilp.linear_logp_backward(f.hidden, f.weight, f.targets, lse, f.grad, f.mask)
    gh, gw = ilp.linear_logp_param_grads(f.hidden, f.weight, f.targets, lse, f.grad, f.mask)
    return [logp, lse, d, gh, gw]


def _logits(c):
    logp, lse = ilp.logp_selected(c.logits, c.targets, c.mask)
    d = ilp.logp_backward(c.logits, c.targets, lse, c.grad, c.mask)
    return [logp, lse, d]


def _bits(ts):
    return [f32bits(t) for t in ts]


def test_two_streams_interleaved(dev):
    f = wl.fused_batch(300, 17000, 136, seed=31, device=dev, w_sigma=0.05, n_masked=20)
    c = wl.logits_batch(500, 40000, 3.0, seed=32, device=dev, n_masked=40)
    ref_f, ref_c = _bits(_fused(f)), _bits(_logits(c))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            of = _fused(f)
        with torch.cuda.stream(s2):
            oc = _logits(c)
        outs.append((of, oc))
    torch.cuda.synchronize()
    for of, oc in outs:
        assert all(torch.equal(a, b) for a, b in zip(_bits(of), ref_f))
        assert all(torch.equal(a, b) for a, b in zip(_bits(oc), ref_c))


def test_host_threads(dev):
    batches = [wl.fused_batch(64 + 37 * i, 3000 + 500 * i, 64, seed=40 + i, device=dev,
                              w_sigma=0.05, n_masked=5) for i in range(4)]
    refs = [_bits(_fused(b)) for b in batches]
    torch.cuda.synchronize()
    results = [None] * len(batches)
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                out = []
                for _ in range(3):
                    out.append(_fused(batches[i]))
            s.synchronize()
            results[i] = out
        except Exception as e:  # surfaced in the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(batches))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for i, outs in enumerate(results):
        assert outs is not None
        for o in outs:
            assert all(torch.equal(a, b) for a, b in zip(_bits(o), refs[i])), i
