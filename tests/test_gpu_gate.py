"""The single-command gate on the GPU: every judgment passes, and a case
replayed from its fixture id alone reproduces its record."""
import pytest

import gate

pytestmark = pytest.mark.gpu


def test_gate_quick_passes():
    report = gate.run_gate(quick=True)
    assert report["status"] == "pass", [c for c in report["cases"] if c["status"] != "pass"][:3]
    for op in ("logp", "linear_logp", "linear_logp_kept"):
        assert set(report["judgments"][op]) == {"forward_accuracy", "forward_invariance",
                                                "gradient_accuracy", "gradient_invariance"}
    assert set(report["judgments"]["linear_logp_params"]) == {"gradient_accuracy",
                                                              "gradient_invariance"}
    assert "gfx950" in report["actual_backend"] and report["fallback"] is None
    assert report["drift_records"] == []
    one = report["cases"][5]
    again = gate.run_gate(quick=True, only=one["fixture_id"])
    assert len(again["cases"]) == 1
    assert again["cases"][0]["status"] == one["status"]
    for k in ("max_abs_error", "n_mismatched", "n_drift_records"):
        if k in one:
            assert again["cases"][0][k] == one[k]
