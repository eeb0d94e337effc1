"""The stored closed-form fixtures (tests/golden/closed_form_rows.json, written
by tests/golden/make_closed_form_rows.py from the oracle): every stored value
equals its closed form, and the oracle as it stands still reproduces it.

The closed forms are those of the selected logprob logp = z_t - ln sum_j
exp z_j and its gradient g (onehot - softmax), the textbook reading of the
operator named by page "[RFC] Batch-Invariant RL Kernel Suite for
Train-Inference Consistency", section "Scope"."""
import json
import math
import os
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_closed_form_rows as mk  # noqa: E402
import oracle  # noqa: E402

GOLDEN = os.path.join(HERE, "golden", "closed_form_rows.json")


def load_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def closed_form(case):
    """(logp, lse, d_target, d_other) from the closed form alone."""
    v, t, g = case["V"], case["target"], case["grad"]
    if case["kind"] == "uniform":
        logp = -math.log(v)
        lse = case["value"] + math.log(v)
        return logp, lse, g * (1 - 1 / v), (-g / v if v > 1 else None)
    if case["kind"] == "pair":
        x = case["x"]
        u = 1 - t
        logp = -math.log1p(math.exp(x[u] - x[t]))
        lse = x[t] - logp
        p_t = math.exp(logp)
        return logp, lse, g * (1 - p_t), -g * (1 - p_t)
    if case["kind"] == "peaked":
        L, base = case["L"], case["base"]
        s = 1 + (v - 1) * math.exp(-L)
        lp_peak, lp_other = -math.log(s), -L - math.log(s)
        logp = lp_peak if t == case["peak_index"] else lp_other
        lse = base + L + math.log(s)
        o = case["dlogits_other_index"]
        p_o = math.exp(lp_peak if o == case["peak_index"] else lp_other)
        return logp, lse, g * (1 - math.exp(logp)), -g * p_o
    raise ValueError(case["kind"])


def close(a, b, tol=1e-12):
    return abs(a - b) <= tol * max(1.0, abs(b))


@pytest.mark.parametrize("case", load_cases(), ids=lambda c: c["name"])
def test_stored_value_is_the_closed_form(case):
    logp, lse, d_t, d_o = closed_form(case)
    assert close(case["logp"], logp), (case["logp"], logp)
    assert close(case["lse"], lse), (case["lse"], lse)
    assert close(case["dlogits_target"], d_t), (case["dlogits_target"], d_t)
    if d_o is not None:
        assert close(case["dlogits_other"], d_o), (case["dlogits_other"], d_o)


def test_oracle_reproduces_the_fixtures():
    for case in load_cases():
        bits = mk.bf16_bits(mk.row_of(case))[None, :]
        t = np.array([case["target"]], dtype=np.int64)
        logp, lse = oracle.logp_selected(bits, t)
        assert logp[0] == case["logp"] and lse[0] == case["lse"], case["name"]
        d = oracle.logp_backward(bits, t, None, lse, np.array([case["grad"]]))[0]
        assert d[case["target"]] == case["dlogits_target"], case["name"]


def test_fixture_cases_match_the_script():
    assert [c["name"] for c in load_cases()] == [c["name"] for c in mk.CASES]
