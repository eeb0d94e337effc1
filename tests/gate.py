"""Single-command gate for the selected-logprob operators on one GPU.

    python tests/gate.py [--quick] [--out report.json] [--replay FIXTURE_ID]

Reports the four judgments that decide "aligned" (page "[WS1 Test] #154
dtype pin + #152 KV path + #153 bwd invariance + #150 chain gate", section
"Sole definition of aligned"): forward_accuracy and gradient_accuracy (the
kernel against the fp64 oracle, within tolerance) and forward_invariance and
gradient_invariance (the kernel against itself under the transform classes
T1-T6, bitwise), each with its own thresholds -- the gradient rows do not
inherit the forward's.  Every failing case carries a drift record in the
schema of page "docs(ws1): batch-invariance contract RFC", section "Drift
Report" (with a stable logical row and the variant row, and stated count
units), and the gate report records the provenance the chain gate asks for
(same page as above, section "Workstream 4 - #150": requested and actual
backend, device, dtype, workload, seed, transform, first failing operator).
There is no fallback: if the native library cannot be loaded the gate fails.

Each case is described by a manifest (operator, workload, seed, transform and
its parameters, generator version); its fixture id is a hash of the manifest
(page "docs(ws1): ...", section "InvarianceFixture", requirement 4), and
``--replay`` re-runs one case from its id alone.
"""

import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

GENERATOR_VERSION = "workloads-1"
THRESHOLDS = {
    "forward_accuracy": {"logp": "2e-5 + 1e-5|r|", "linear_logp": "2e-3",
                         "linear_logp_kept": "2e-3"},
    "gradient_accuracy": {"logp": "1e-3", "linear_logp": "1e-3", "linear_logp_kept": "1e-3",
                          "linear_logp_params": "min(1e-3, 1e-4 sum|D||W| + 1e-5) (grad_hidden), "
                                                "min(1e-3, 1e-4 sum|D||h| + 1e-5) (grad_weight)"},
    "forward_invariance": {"atol": 0.0, "rtol": 0.0},
    "gradient_invariance": {"atol": 0.0, "rtol": 0.0},
}
# linear_logp_kept: the fused operator with its fp32 logits kept by the
# forward and its backward computed from them (the same chain entry)
CHAIN_INDEX = {"logp": 8, "linear_logp": 7, "linear_logp_kept": 7, "linear_logp_params": 7}
OPERATORS = ("logp", "linear_logp", "linear_logp_kept", "linear_logp_params")


def fixture_id(man):
    blob = json.dumps(man, sort_keys=True).encode()
    return f"{man['operator']}-{hashlib.sha256(blob).hexdigest()[:12]}"


def case_list(quick):
    """Manifests of every case of the gate, in a fixed order."""
    cases = []
    logits_wl = [("logits_small", {}), ("logits_varlen", {})]
    if not quick:
        logits_wl.append(("logits_large_rows", {"n": 512}))
    for wl_name, wl_args in logits_wl:
        cases.append({"operator": "logp", "judgment": "forward_accuracy", "workload": wl_name,
                      "workload_args": wl_args, "seed": 0})
        cases.append({"operator": "logp", "judgment": "gradient_accuracy", "workload": wl_name,
                      "workload_args": wl_args, "seed": 0})
        for t in (("T1", {"size": 1, "start": 3}), ("T1", {"size": 7, "start": 1}),
                  ("T2", {"seed": 1}), ("T3", {"keep_every": 5, "seed": 2}),
                  ("T4", {"left": 2, "right": 3, "every": 16, "seed": 3}),
                  ("T5", {"chunk": 1}), ("T5", {"chunk": 5}), ("T6", {"compacted": True})):
            for j in ("forward_invariance", "gradient_invariance"):
                cases.append({"operator": "logp", "judgment": j, "workload": wl_name,
                              "workload_args": wl_args, "seed": 0,
                              "transform": {"class": t[0], **t[1]}})
    fused = [("fused_small", {"n": 96, "v": 1300, "h": 256})]
    if not quick:
        fused.append(("fused_small", {"n": 300, "v": 4000, "h": 512}))
    for wl_name, wl_args in fused:
        for j in ("forward_accuracy", "gradient_accuracy"):
            cases.append({"operator": "linear_logp", "judgment": j, "workload": wl_name,
                          "workload_args": wl_args, "seed": 0})
        for t in (("T1", {"size": 1, "start": 5}), ("T1", {"size": 33, "start": 7}),
                  ("T2", {"seed": 1}), ("T4", {"left": 3, "right": 1, "every": 40, "seed": 4}),
                  ("T5", {"chunk": 32})):
            for j in ("forward_invariance", "gradient_invariance"):
                cases.append({"operator": "linear_logp", "judgment": j, "workload": wl_name,
                              "workload_args": wl_args, "seed": 0,
                              "transform": {"class": t[0], **t[1]}})
    # the same operator with the logits kept by the forward: the first fused
    # workload, all four judgments
    wl_name, wl_args = fused[0]
    for j in ("forward_accuracy", "gradient_accuracy"):
        cases.append({"operator": "linear_logp_kept", "judgment": j, "workload": wl_name,
                      "workload_args": wl_args, "seed": 0})
    for t in (("T1", {"size": 1, "start": 5}), ("T2", {"seed": 1}),
              ("T4", {"left": 3, "right": 1, "every": 40, "seed": 4}), ("T5", {"chunk": 32})):
        for j in ("forward_invariance", "gradient_invariance"):
            cases.append({"operator": "linear_logp_kept", "judgment": j, "workload": wl_name,
                          "workload_args": wl_args, "seed": 0,
                          "transform": {"class": t[0], **t[1]}})
    # parameter gradients of the fused path: accuracy of both outputs; bitwise
    # invariance of grad_hidden rows; grad_weight over the same complete sample
    # set (masked rows appended after the batch) bitwise
    for wl_name, wl_args in fused:
        cases.append({"operator": "linear_logp_params", "judgment": "gradient_accuracy",
                      "workload": wl_name, "workload_args": wl_args, "seed": 0})
        for t in (("T1", {"size": 1, "start": 5}), ("T2", {"seed": 1}),
                  ("T4", {"left": 3, "right": 1, "every": 40, "seed": 4}), ("T5", {"chunk": 32}),
                  ("T4", {"left": 0, "right": 9, "every": 0, "seed": 5, "output": "grad_weight"})):
            cases.append({"operator": "linear_logp_params", "judgment": "gradient_invariance",
                          "workload": wl_name, "workload_args": wl_args, "seed": 0,
                          "transform": {"class": t[0], **t[1]}})
    for c in cases:
        c["generator"] = GENERATOR_VERSION
        c["fixture_id"] = fixture_id({k: v for k, v in c.items() if k != "fixture_id"})
    return cases


class Runner:
    """Builds inputs for a manifest and runs one case on the GPU."""

    def __init__(self):
        import torch

        import invariant_logprob_amd as ilp
        self.torch = torch
        self.ilp = ilp
        if not torch.cuda.is_available():
            raise RuntimeError("the gate needs a GPU; a CPU-only run cannot certify it")
        self.dev = torch.device("cuda:0")
        ilp.load_library()   # raises when the native library is missing: no fallback
        self._cache = {}

    # -- inputs -----------------------------------------------------------
    def batch(self, man):
        key = (man["workload"], json.dumps(man["workload_args"], sort_keys=True), man["seed"])
        if key in self._cache:
            return self._cache[key]
        from invariant_logprob_amd import workloads as wl
        a = man["workload_args"]
        if man["workload"] == "logits_small":
            b = wl.logits_small(man["seed"], self.dev)
            base = {"x": b.logits, "targets": b.targets, "mask": b.mask, "grad": b.grad}
            shared = {}
        elif man["workload"] == "logits_varlen":
            import invariance as inv
            b = wl.logits_varlen(man["seed"], self.dev)
            n = min(b.logits.shape[0], 160)
            base = {"x": b.logits[:n], "targets": b.targets[:n], "mask": b.mask[:n],
                    "grad": b.grad[:n]}
            # drift records name (sequence, token position) of the packing
            shared = {"positions": inv.canonical_positions(n, b.seq_lens)}
        elif man["workload"] == "logits_large_rows":
            b = wl.logits_batch(a["n"], 151936, 4.0, man["seed"], self.dev,
                                n_masked=int(round(0.15 * a["n"])))
            base = {"x": b.logits, "targets": b.targets, "mask": b.mask, "grad": b.grad}
            shared = {}
        elif man["workload"] == "fused_small":
            b = wl.fused_batch(a["n"], a["v"], a["h"], man["seed"], self.dev, w_sigma=0.05,
                               n_masked=a["n"] // 12)
            base = {"x": b.hidden, "targets": b.targets, "mask": b.mask, "grad": b.grad}
            shared = {"weight": b.weight}
        else:
            raise ValueError(man["workload"])
        self._cache[key] = (base, shared)
        return base, shared

    def filler(self, man, shared):
        torch = self.torch
        from invariant_logprob_amd import workloads as wl
        dev = self.dev
        if man["operator"] == "logp":
            v = self.batch(man)[0]["x"].shape[1]

            def f(n, seed):
                x, t = wl.neighbour_rows(n, v, seed, device=dev)
                g = torch.Generator(device=dev).manual_seed(seed)
                return {"x": x, "targets": t, "mask": torch.ones(n, dtype=torch.uint8, device=dev),
                        "grad": torch.randn(n, generator=g, device=dev)}
        else:
            h = shared["weight"].shape[1]
            v = shared["weight"].shape[0]

            def f(n, seed):
                g = torch.Generator(device=dev).manual_seed(seed)
                return {"x": (torch.randn((n, h), generator=g, device=dev) * 3).to(torch.bfloat16),
                        "targets": torch.randint(0, v, (n,), generator=g, device=dev),
                        "mask": torch.ones(n, dtype=torch.uint8, device=dev),
                        "grad": torch.randn(n, generator=g, device=dev)}
        return f

    # -- the operator under test ------------------------------------------
    def run_op(self, man, shared, batch, backward, want_weight=False):
        ilp = self.ilp
        if man["operator"] == "linear_logp_params":
            w = shared["weight"]
            _, lse = ilp.linear_logp(batch["x"], w, batch["targets"], batch["mask"])
            gh, gw = ilp.linear_logp_param_grads(batch["x"], w, batch["targets"], lse,
                                                 batch["grad"], batch["mask"],
                                                 want_weight=want_weight)
            return {"grad_weight": gw} if want_weight else {"grad_hidden": gh}
        if man["operator"] == "logp":
            logp, lse = ilp.logp_selected(batch["x"], batch["targets"], batch["mask"])
            out = {"logp": logp, "lse": lse}
            if backward:
                out = {"dlogits": ilp.logp_backward(batch["x"], batch["targets"], lse,
                                                    batch["grad"], batch["mask"])}
        elif man["operator"] == "linear_logp_kept":
            w = shared["weight"]
            logp, lse, z = ilp.linear_logp_with_logits(batch["x"], w, batch["targets"],
                                                       batch["mask"])
            out = {"logp": logp, "lse": lse}
            if backward:
                out = {"dlogits": ilp.logp_backward(z, batch["targets"], lse, batch["grad"],
                                                    batch["mask"], out=z)}
        else:
            w = shared["weight"]
            logp, lse = ilp.linear_logp(batch["x"], w, batch["targets"], batch["mask"])
            out = {"logp": logp, "lse": lse}
            if backward:
                out = {"dlogits": ilp.linear_logp_backward(batch["x"], w, batch["targets"], lse,
                                                           batch["grad"], batch["mask"])}
        return out

    # -- one case ---------------------------------------------------------
    def run_case(self, man):
        import numpy as np

        import invariance as inv
        import oracle
        torch = self.torch
        base, shared = self.batch(man)
        backward = man["judgment"].startswith("gradient")
        rec = {"fixture_id": man["fixture_id"], "operator": man["operator"],
               "chain_index": CHAIN_INDEX[man["operator"]], "judgment": man["judgment"],
               "workload": man["workload"], "workload_args": man["workload_args"],
               "seed": man["seed"], "transform": man.get("transform")}
        if man["operator"] == "linear_logp_params":
            return self.run_params_case(man, shared, base, rec)
        if man["judgment"].endswith("accuracy"):
            out = self.run_op(man, shared, base, backward)
            torch.cuda.synchronize()
            bits = lambda t: t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
            m = base["mask"].cpu().numpy()
            act = m.astype(bool)
            t = base["targets"].cpu().numpy()
            # gradient references are end to end: the oracle's own lse,
            # never a value the GPU produced
            if man["operator"] == "logp":
                rlogp, rlse = oracle.logp_selected(bits(base["x"]), t, m)
                if backward:
                    ref = {"dlogits": oracle.logp_backward(bits(base["x"]), t, m, rlse,
                                                           base["grad"].cpu().numpy())}
                else:
                    ref = {"logp": rlogp, "lse": rlse}
                tol = (lambda r: 2e-5 + 1e-5 * np.abs(r)) if not backward else (lambda r: 1e-3)
            else:
                hb, wb = bits(base["x"]), bits(shared["weight"])
                rlogp, rlse = oracle.linear_logp(hb, wb, t, m)
                if backward:
                    ref = {"dlogits": oracle.linear_logp_backward(hb, wb, t, m, rlse,
                                                                  base["grad"].cpu().numpy())}
                else:
                    ref = {"logp": rlogp, "lse": rlse}
                tol = (lambda r: 2e-3) if not backward else (lambda r: 1e-3)
            worst = {"max_abs_error": 0.0, "max_rel_error": 0.0, "n_mismatched": 0, "n_compared": 0}
            first = None
            for k, r in ref.items():
                g = out[k].cpu().numpy().astype(np.float64)
                if g.ndim == 1:
                    g, r = g[act], r[act]
                err = np.abs(g - r)
                bad = ~(err <= tol(r))
                worst["max_abs_error"] = max(worst["max_abs_error"], float(np.nanmax(err)) if err.size else 0.0)
                rel = err / np.maximum(np.abs(r), 1e-30)
                worst["max_rel_error"] = max(worst["max_rel_error"], float(np.nanmax(rel)) if rel.size else 0.0)
                worst["n_mismatched"] += int(bad.sum())
                worst["n_compared"] += int(bad.size)
                if bad.any() and first is None:
                    first = {"output": k, "index": [int(i) for i in np.argwhere(bad)[0]]}
            rec.update(worst)
            rec["units"] = "output elements"
            rec["status"] = "pass" if worst["n_mismatched"] == 0 else "fail"
            rec["threshold"] = THRESHOLDS[man["judgment"]][man["operator"]]
            rec["first_mismatch"] = first
            return rec, []
        # invariance: the kernel against itself under the declared transform
        t = man["transform"]
        filler = self.filler(man, shared)
        cls = t["class"]
        n = inv.nrows(base)
        if cls == "T1":
            calls, row_map = inv.t1_population(base, t["size"], t["start"])
        elif cls == "T2":
            calls, row_map = inv.t2_position(base, t["seed"])
        elif cls == "T3":
            calls, row_map = inv.t3_neighbours(base, list(range(0, n, t["keep_every"])), filler,
                                               t["seed"])
        elif cls == "T4":
            calls, row_map = inv.t4_padding(base, filler, t["seed"], t["left"], t["right"],
                                            t["every"])
        elif cls == "T5":
            calls, row_map = inv.t5_schedule(base, t["chunk"])
        elif cls == "T6":
            calls, row_map = inv.t6_compacted(base)
        else:
            raise ValueError(cls)
        run = lambda b: self.run_op(man, shared, b, backward)
        manifest = {"operator": man["operator"], "chain_index": CHAIN_INDEX[man["operator"]],
                    "transform": {**t, "name": inv.TRANSFORM_NAMES[cls]}, "seed": man["seed"],
                    "device": str(self.dev), "direction": "backward" if backward else "forward",
                    "launch": {"calls": len(calls), "rows": [inv.nrows(c) for c in calls][:4]}}
        recs, _ = inv.check(run, base, calls, row_map, manifest,
                            positions=shared.get("positions"))
        for r in recs:
            r["fixture_id"] = man["fixture_id"]
        rec.update({"status": "pass" if not recs else "fail",
                    "threshold": THRESHOLDS[man["judgment"]],
                    "n_drift_records": len(recs)})
        return rec, recs


def _params_case(self, man, shared, base, rec):
    """Parameter gradients: accuracy of grad_hidden and grad_weight against
    the oracle's end-to-end gradients (its own lse) within min(1e-3, 1e-4 S +
    1e-5), S the absolute sum of the summed terms; invariance of grad_hidden
    rows (harness) or of grad_weight over the same complete sample set (masked
    rows appended), bitwise."""
    import numpy as np

    import invariance as inv
    import oracle
    torch = self.torch
    ilp = self.ilp
    w = shared["weight"]
    if man["judgment"] == "gradient_accuracy":
        _, lse = ilp.linear_logp(base["x"], w, base["targets"], base["mask"])
        gh, gw = ilp.linear_logp_param_grads(base["x"], w, base["targets"], lse, base["grad"],
                                             base["mask"])
        torch.cuda.synchronize()
        bits = lambda t: t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        hb, wb = bits(base["x"]), bits(w)
        t = base["targets"].cpu().numpy()
        m = base["mask"].cpu().numpy()
        g = base["grad"].cpu().numpy()
        rgh, rgw = oracle.linear_param_grads(hb, wb, t, m, None, g)
        d_abs = np.abs(oracle.linear_logp_backward(hb, wb, t, m, None, g))
        bounds = {"grad_hidden": d_abs @ np.abs(oracle.bf16_to_f64(wb)),
                  "grad_weight": d_abs.T @ np.abs(oracle.bf16_to_f64(hb))}
        worst = {"max_abs_error": 0.0, "max_rel_error": 0.0, "n_mismatched": 0, "n_compared": 0}
        first = None
        for k, got, ref in (("grad_hidden", gh, rgh), ("grad_weight", gw, rgw)):
            got = got.cpu().numpy().astype(np.float64)
            err = np.abs(got - ref)
            bad = ~(err <= np.minimum(1e-3, 1e-4 * bounds[k] + 1e-5))
            worst["max_abs_error"] = max(worst["max_abs_error"], float(np.nanmax(err)))
            rel = err / np.maximum(np.abs(ref), 1e-30)
            worst["max_rel_error"] = max(worst["max_rel_error"], float(np.nanmax(rel)))
            worst["n_mismatched"] += int(bad.sum())
            worst["n_compared"] += int(bad.size)
            if bad.any() and first is None:
                first = {"output": k, "index": [int(i) for i in np.argwhere(bad)[0]]}
        rec.update(worst)
        rec.update({"units": "output elements", "first_mismatch": first,
                    "status": "pass" if worst["n_mismatched"] == 0 else "fail",
                    "threshold": THRESHOLDS["gradient_accuracy"]["linear_logp_params"]})
        return rec, []
    tr = man["transform"]
    filler = self.filler(man, shared)
    cls = tr["class"]
    if cls == "T1":
        calls, row_map = inv.t1_population(base, tr["size"], tr["start"])
    elif cls == "T2":
        calls, row_map = inv.t2_position(base, tr["seed"])
    elif cls == "T4":
        calls, row_map = inv.t4_padding(base, filler, tr["seed"], tr["left"], tr["right"],
                                        tr["every"])
    elif cls == "T5":
        calls, row_map = inv.t5_schedule(base, tr["chunk"])
    else:
        raise ValueError(cls)
    manifest = {"operator": man["operator"], "chain_index": CHAIN_INDEX[man["operator"]],
                "transform": {**tr, "name": inv.TRANSFORM_NAMES[cls]}, "seed": man["seed"],
                "device": str(self.dev), "direction": "backward",
                "launch": {"calls": len(calls), "rows": [inv.nrows(c) for c in calls][:4]}}
    if tr.get("output") == "grad_weight":
        # the same complete sample set, the padding rows masked: one call each
        assert len(calls) == 1
        a = self.run_op(man, shared, base, True, want_weight=True)["grad_weight"]
        b = self.run_op(man, shared, calls[0], True, want_weight=True)["grad_weight"]
        torch.cuda.synchronize()
        ia = a.contiguous().view(torch.int32)
        ib = b.contiguous().view(torch.int32)
        diff = (ia != ib)
        recs = []
        if bool(diff.any()):
            first = [int(i) for i in torch.nonzero(diff)[0].cpu()]
            recs.append({"relation": "I", "status": "fail", "fixture_id": man["fixture_id"],
                         "operator": man["operator"], "transform": manifest["transform"],
                         "output": "grad_weight", "n_mismatched": int(diff.sum()),
                         "units": "output elements", "first_mismatch": first})
    else:
        run = lambda bt: self.run_op(man, shared, bt, True)
        recs, _ = inv.check(run, base, calls, row_map, manifest)
        for r in recs:
            r["fixture_id"] = man["fixture_id"]
    rec.update({"status": "pass" if not recs else "fail",
                "threshold": THRESHOLDS[man["judgment"]], "n_drift_records": len(recs)})
    return rec, recs


Runner.run_params_case = _params_case


def run_gate(quick=False, only=None):
    import torch
    runner = Runner()
    cases = case_list(quick)
    if only is not None:
        cases = [c for c in cases if c["fixture_id"] == only]
        if not cases:
            raise SystemExit(f"unknown fixture id {only}")
    t0 = time.time()
    results, drift = [], []
    for man in cases:
        rec, recs = runner.run_case(man)
        results.append(rec)
        drift += recs
    table = {}
    for op in OPERATORS:
        for j in ("forward_accuracy", "forward_invariance", "gradient_accuracy", "gradient_invariance"):
            sel = [r for r in results if r["operator"] == op and r["judgment"] == j]
            if sel:
                table.setdefault(op, {})[j] = {
                    "status": "pass" if all(r["status"] == "pass" for r in sel) else "fail",
                    "cases": len(sel), "threshold": THRESHOLDS[j] if "invariance" in j
                    else THRESHOLDS[j][op]}
    failing = sorted({r["chain_index"] for r in results if r["status"] == "fail"})
    report = {
        "gate": "selected-logprob operators",
        "requested_backend": "hip-gfx950",
        "actual_backend": runner.ilp.build_info(),
        "fallback": None,
        "device": torch.cuda.get_device_name(runner.dev),
        "dtype": "bfloat16 inputs, float32 outputs",
        "generator": GENERATOR_VERSION,
        "judgments": table,
        "first_failing_chain_index": failing[0] if failing else None,
        "status": "pass" if all(r["status"] == "pass" for r in results) else "fail",
        "cases": results,
        "drift_records": drift,
        "seconds": round(time.time() - t0, 2),
    }
    return report


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--quick", action="store_true")
    ap.add_argument("--out", default=None)
    ap.add_argument("--replay", default=None, help="re-run one case by fixture id")
    ap.add_argument("--list", action="store_true", help="print the case manifests")
    args = ap.parse_args()
    if args.list:
        print(json.dumps(case_list(args.quick), indent=1))
        return 0
    report = run_gate(args.quick, args.replay)
    text = json.dumps(report, indent=1, default=str)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    summary = {"status": report["status"], "judgments": report["judgments"],
               "actual_backend": report["actual_backend"], "cases": len(report["cases"]),
               "drift_records": len(report["drift_records"]), "seconds": report["seconds"]}
    print(json.dumps(summary, indent=1))
    return 0 if report["status"] == "pass" else 1


if __name__ == "__main__":
    sys.exit(main())
