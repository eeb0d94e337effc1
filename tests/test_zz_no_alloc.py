"""The allocation-free fused forward (rlk_linear_logp_noalloc) against the
workspace entry point (rlk_linear_logp), both through the C ABI: two calls in
a row, the first at the size limit of the library's 32 MiB per-GPU array, the
second smaller (so the array holds the first call's contents), then a
five-row batch (the small-batch forward), each bit-identical to
rlk_linear_logp's output on the same inputs; the 300-row one also against the
fp64 oracle within the fused tolerance."""
import numpy as np
import pytest
import torch

import invariant_logprob_amd as ilp
import oracle
from gpu_util import TOL_FUSED, assert_close, bits16, f32bits, require_gpu
from invariant_logprob_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    ilp.load_library()
    return d


def _both(b):
    n = b.hidden.shape[0]
    lp = torch.full((n,), float("nan"), device=b.hidden.device)
    ls = torch.full((n,), float("nan"), device=b.hidden.device)
    lp_n, ls_n = ilp.linear_logp_noalloc(b.hidden, b.weight, b.targets, b.mask, logp=lp, lse=ls)
    lp_w, ls_w = ilp.linear_logp(b.hidden, b.weight, b.targets, b.mask)
    torch.cuda.synchronize()
    assert lp_n.data_ptr() == lp.data_ptr() and ls_n.data_ptr() == ls.data_ptr()
    return lp_n, ls_n, lp_w, ls_w


def test_noalloc_matches_workspace_entry_point(dev):
    # 7055 rows at V = 151936: 7055 x 594 partials + target logits = 32 MiB
    big = wl.fused_batch(7055, 151936, 64, seed=51, device=dev, w_sigma=0.05, n_masked=700)
    assert ilp.linear_logp_workspace_size(7055, 151936, 64) <= 32 << 20
    lp_n, ls_n, lp_w, ls_w = _both(big)
    assert torch.equal(f32bits(lp_n), f32bits(lp_w)) and torch.equal(f32bits(ls_n), f32bits(ls_w))
    del big
    # a smaller problem right after: the array still holds the first call's
    # partials, none of which may leak into this one
    small = wl.fused_batch(300, 2600, 256, seed=52, device=dev, w_sigma=0.05, n_masked=30)
    lp_n, ls_n, lp_w, ls_w = _both(small)
    assert torch.equal(f32bits(lp_n), f32bits(lp_w)) and torch.equal(f32bits(ls_n), f32bits(ls_w))
    rlogp, rlse = oracle.linear_logp(bits16(small.hidden), bits16(small.weight),
                                     small.targets.cpu().numpy(), small.mask.cpu().numpy())
    act = small.mask.cpu().numpy().astype(bool)
    assert_close(lp_n.cpu().numpy(), rlogp, TOL_FUSED, "noalloc logp", act)
    assert_close(ls_n.cpu().numpy(), rlse, TOL_FUSED, "noalloc lse", act)
    assert bool((f32bits(lp_n)[torch.from_numpy(~act)] == 0).all())
    # and a batch small enough for the small-batch forward
    tiny = wl.fused_batch(5, 2600, 256, seed=54, device=dev, w_sigma=0.05)
    lp_n, ls_n, lp_w, ls_w = _both(tiny)
    assert torch.equal(f32bits(lp_n), f32bits(lp_w)) and torch.equal(f32bits(ls_n), f32bits(ls_w))


def test_noalloc_refuses_beyond_its_array(dev):
    b = wl.fused_batch(7056, 151936, 64, seed=53, device=dev, w_sigma=0.05)
    with pytest.raises(ilp.RlkError) as e:
        ilp.linear_logp_noalloc(b.hidden, b.weight, b.targets)
    assert e.value.status == 2
