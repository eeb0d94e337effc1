"""The gate's case manifests (CPU only): fixed order, unique content-derived
fixture ids, the four judgments present for every operator."""
import json
import os
import subprocess
import sys

import gate


def test_fixture_ids_unique_and_stable():
    a = gate.case_list(quick=False)
    b = gate.case_list(quick=False)
    assert [c["fixture_id"] for c in a] == [c["fixture_id"] for c in b]
    ids = [c["fixture_id"] for c in a]
    assert len(ids) == len(set(ids))
    for c in a:
        man = {k: v for k, v in c.items() if k != "fixture_id"}
        assert gate.fixture_id(man) == c["fixture_id"]


def test_every_judgment_is_covered():
    cases = gate.case_list(quick=True)
    for op in ("logp", "linear_logp", "linear_logp_kept"):
        js = {c["judgment"] for c in cases if c["operator"] == op}
        assert js == {"forward_accuracy", "forward_invariance", "gradient_accuracy",
                      "gradient_invariance"}
    classes = {c["transform"]["class"] for c in cases if "transform" in c}
    assert classes == {"T1", "T2", "T3", "T4", "T5", "T6"}


def test_list_command_runs_without_gpu():
    here = os.path.dirname(os.path.abspath(__file__))
    r = subprocess.run([sys.executable, os.path.join(here, "gate.py"), "--list", "--quick"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    assert len(json.loads(r.stdout)) == len(gate.case_list(quick=True))
