"""The GPU logits path on the stored closed-form rows
(tests/golden/closed_form_rows.json): selected logprob and log-sum-exp within
|d| <= 2e-5 + 1e-5 |r|, the logits gradient within 1e-3, through the C ABI."""
import json
import os

import pytest
import torch

import invariant_logprob_amd as ilp
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "closed_form_rows.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _row(case, dev):
    """The case's bf16 row as a [1, V] view of a padded buffer."""
    v = case["V"]
    buf = torch.zeros((1, (v + 7) // 8 * 8), dtype=torch.float32, device=dev)
    if case["kind"] == "uniform":
        buf[0, :v] = case["value"]
    elif case["kind"] == "pair":
        buf[0, 0], buf[0, 1] = case["x"]
    else:
        buf[0, :v] = case["base"]
        buf[0, case["peak_index"]] += case["L"]
    return buf.to(torch.bfloat16)[:, :v]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_logits_path_on_closed_form_rows(case):
    dev = require_gpu()
    x = _row(case, dev)
    t = torch.tensor([case["target"]], dtype=torch.int64, device=dev)
    logp, lse = ilp.logp_selected(x, t)
    g = torch.tensor([case["grad"]], dtype=torch.float32, device=dev)
    d = ilp.logp_backward(x, t, lse, g)
    torch.cuda.synchronize()
    for got, ref in ((float(logp[0]), case["logp"]), (float(lse[0]), case["lse"])):
        assert abs(got - ref) <= 2e-5 + 1e-5 * abs(ref), (case["name"], got, ref)
    assert abs(float(d[0, case["target"]]) - case["dlogits_target"]) <= 1e-3
    if case["dlogits_other"] is not None:
        assert abs(float(d[0, case["dlogits_other_index"]]) - case["dlogits_other"]) <= 1e-3
