"""Writes closed_form_rows.json: rows whose selected logprob, log-sum-exp and
logits gradient have closed forms, with the expected values computed by the
fp64 oracle (this script calls nothing but oracle/ and the standard library).

    python tests/golden/make_closed_form_rows.py

The closed forms follow from the definition logp = z_t - ln sum_j exp z_j and
its derivative g (onehot - softmax) (the textbook reading of the operator the
page "[RFC] Batch-Invariant RL Kernel Suite for Train-Inference Consistency"
names in its "Scope" section); tests/test_golden.py checks every stored value
against its closed form, so the file is pinned by the mathematics, not by the
oracle alone.  Every input value is exactly representable in bf16.
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402


def bf16_bits(x):
    """Raw bf16 bits of float64 values that bf16 represents exactly."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value not exactly representable in bf16")
    return (u >> 16).astype(np.uint16)


def row_of(case):
    """The case's logits row as float64 [V]."""
    v = case["V"]
    if case["kind"] == "uniform":
        return np.full(v, case["value"], dtype=np.float64)
    if case["kind"] == "pair":
        return np.asarray(case["x"], dtype=np.float64)
    if case["kind"] == "peaked":
        x = np.full(v, case["base"], dtype=np.float64)
        x[case["peak_index"]] += case["L"]
        return x
    raise ValueError(case["kind"])


CASES = []
for v in (1, 2, 1024, 32000, 128256, 151936):
    for c in (0.0, 3.5, -7.25):
        CASES.append({"name": f"uniform_V{v}_c{c}", "kind": "uniform", "V": v, "value": c,
                      "target": (v * 7) // 11, "grad": 0.75,
                      "closed_form": "logp = -ln V; lse = c + ln V; dlogits = g ([j == t] - 1/V)"})
for x0, x1 in ((0.0, 0.0), (1.0, -1.0), (-3.5, 2.25), (20.0, -20.0), (0.5, 8.0)):
    for t in (0, 1):
        CASES.append({"name": f"pair_{x0}_{x1}_t{t}", "kind": "pair", "V": 2, "x": [x0, x1],
                      "target": t, "grad": -1.5,
                      "closed_form": "logp_t = -log1p(exp(x_u - x_t)) for the other entry u; "
                                     "dlogits_t = g (1 - exp(logp_t))"})
for v, L in ((1000, 1.0), (1000, 5.0), (32000, 20.0), (151936, 12.0)):
    for t_is_peak in (True, False):
        peak = (v * 3) // 7
        CASES.append({"name": f"peaked_V{v}_L{L}_{'peak' if t_is_peak else 'other'}",
                      "kind": "peaked", "V": v, "base": -2.0, "L": L, "peak_index": peak,
                      "target": peak if t_is_peak else peak - 1, "grad": 1.25,
                      "closed_form": "logp_peak = -ln(1 + (V - 1) e^-L); "
                                     "logp_other = -L - ln(1 + (V - 1) e^-L)"})


def main():
    out = []
    for case in CASES:
        x = row_of(case)
        bits = bf16_bits(x)[None, :]
        t = np.array([case["target"]], dtype=np.int64)
        logp, lse = oracle.logp_selected(bits, t)
        d = oracle.logp_backward(bits, t, None, lse, np.array([case["grad"]]))[0]
        rec = dict(case)
        rec["logp"] = float(logp[0])
        rec["lse"] = float(lse[0])
        rec["dlogits_target"] = float(d[case["target"]])
        other = 0 if case["target"] != 0 else case["V"] - 1
        rec["dlogits_other_index"] = int(other)
        rec["dlogits_other"] = float(d[other]) if case["V"] > 1 else None
        out.append(rec)
    doc = {"description": "single logits rows with closed-form selected logprob, log-sum-exp "
                          "and gradient; expected values from the fp64 oracle",
           "generated_by": "tests/golden/make_closed_form_rows.py",
           "cases": out}
    with open(os.path.join(HERE, "closed_form_rows.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(f"wrote {len(out)} cases")


if __name__ == "__main__":
    main()
