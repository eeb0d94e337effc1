"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is a fresh copy of the oracle module with one plausible error
patched in (a dropped term, a wrong sign or index, a transposed operand, a
wrong logarithm base, an ignored mask).  The real oracle passes every pin
(test_oracle_pins); these tests show the pins would notice such mistakes.
"""
import importlib.util
import os

import numpy as np
import pytest

from oracle_pins import ALL_PINS

ORACLE_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "oracle", "logprob_oracle.py")


def fresh_oracle(tag):
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{tag}", ORACLE_FILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _lse_factory(variant):
    def lse(x):
        x = np.asarray(x, dtype=np.float64)
        m = np.max(x, axis=1)
        with np.errstate(all="ignore"):
            if variant == "sign":
                return m - np.log(np.sum(np.exp(x - m[:, None]), axis=1))
            if variant == "no_shift":
                return np.log(np.sum(np.exp(x), axis=1))
            if variant == "log2":
                return m + np.log2(np.sum(np.exp(x - m[:, None]), axis=1))
            if variant == "drop_max":
                return np.log(np.sum(np.exp(x - m[:, None]), axis=1))
            if variant == "mean_not_sum":
                return m + np.log(np.mean(np.exp(x - m[:, None]), axis=1))
        raise AssertionError(variant)
    return lse


def make_mutant(name):
    o = fresh_oracle(name)
    if name in ("sign", "no_shift", "log2", "drop_max", "mean_not_sum"):
        o.logsumexp_rows = _lse_factory(name)
    elif name == "gather_off_by_one":
        orig = o.selected_logp_from_f64

        def f(x, targets, mask=None):
            t = np.asarray(targets, dtype=np.int64)
            v = np.asarray(x).shape[1]
            return orig(x, (t + 1) % v if v > 1 else t, mask)
        o.selected_logp_from_f64 = f
    elif name == "decode_as_fp16":
        o.bf16_to_f64 = lambda b: np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)
    elif name == "weight_transposed":
        def ll(hb, wb):
            h = o.bf16_to_f64(hb)
            w = o.bf16_to_f64(wb)
            v, hh = w.shape
            return h @ w.reshape(hh, v)  # reads [V,H] memory as if it were [H,V]
        o.linear_logits = ll
        orig_lp = o.linear_logp

        def lp(hb, wb, t, mask=None, block_rows=256):
            return o.selected_logp_from_f64(ll(hb, wb), t, mask)
        o.linear_logp = lp
        del orig_lp
    elif name == "mask_ignored":
        orig = o.selected_logp_from_f64

        def f(x, targets, mask=None):
            t = np.asarray(targets, dtype=np.int64).copy()
            v = np.asarray(x).shape[1]
            t = np.where((t < 0) | (t >= v), 0, t)
            return orig(x, t, None)
        o.selected_logp_from_f64 = f
    elif name in ("bwd_sign", "bwd_no_g", "bwd_no_onehot", "bwd_no_lse"):
        def b(x, targets, mask, lse, g):
            x = np.asarray(x, dtype=np.float64)
            n, v = x.shape
            t = np.asarray(targets, dtype=np.int64)
            act = np.ones(n, bool) if mask is None else np.asarray(mask).astype(bool)
            g = np.asarray(g, dtype=np.float64).reshape(n)
            ls = np.asarray(lse, dtype=np.float64).reshape(n)
            d = np.zeros((n, v))
            for i in np.nonzero(act)[0]:
                p = np.exp(x[i] - (0.0 if name == "bwd_no_lse" else ls[i]))
                oh = np.zeros(v)
                if name != "bwd_no_onehot":
                    oh[t[i]] = 1.0
                gi = 1.0 if name == "bwd_no_g" else g[i]
                d[i] = gi * ((p - oh) if name == "bwd_sign" else (oh - p))
            return d
        o.logp_backward_from_f64 = b
    elif name == "entropy_sign":
        clean = fresh_oracle("clean_entropy")
        o.entropy_from_f64 = lambda x, mask=None: -clean.entropy_from_f64(x, mask)
        o.entropy = lambda b, mask=None, block_rows=256: -clean.entropy(b, mask)
    elif name == "entropy_no_p":
        def ent(x, mask=None):
            x = np.asarray(x, dtype=np.float64)
            n = x.shape[0]
            act = np.ones(n, bool) if mask is None else np.asarray(mask).astype(bool)
            out = np.zeros(n)
            lse = o.logsumexp_rows(x)
            with np.errstate(all="ignore"):
                out[act] = -np.sum(x[act] - lse[act, None], axis=1) / x.shape[1]
            return out
        o.entropy_from_f64 = ent
        o.entropy = lambda b, mask=None, block_rows=256: ent(o.bf16_to_f64(b), mask)
    elif name == "log_softmax_no_lse":
        o.log_softmax_from_f64 = lambda x, mask=None: np.asarray(x, dtype=np.float64) - np.max(x, axis=1, keepdims=True)
        o.log_softmax = lambda b, mask=None: o.log_softmax_from_f64(o.bf16_to_f64(b), mask)
    elif name in ("loss_max_not_min", "loss_grad_ignores_clip", "kl_sign"):
        clean = fresh_oracle("clean_loss")

        def tl(logp, logp_old, adv, mask=None, logp_ref=None, eps_lo=0.2, eps_hi=0.2, beta=0.0):
            out = clean.token_losses(logp, logp_old, adv, mask, logp_ref, eps_lo, eps_hi, beta)
            lp = np.asarray(logp, dtype=np.float64)
            r = np.exp(lp - np.asarray(logp_old, dtype=np.float64))
            a = np.asarray(adv, dtype=np.float64)
            if name == "loss_max_not_min":
                out["loss"] = -np.maximum(r * a, np.clip(r, 1 - eps_lo, 1 + eps_hi) * a) + beta * out["kl"]
            elif name == "loss_grad_ignores_clip":
                g = -a * r
                if logp_ref is not None:
                    g = g + beta * (1 - np.exp(np.asarray(logp_ref) - lp))
                out["grad"] = g
            else:
                out["kl"] = -out["kl"]
            return out
        o.token_losses = tl
    elif name in ("pgrad_sign", "pgrad_h_rows_reversed", "pgrad_w_no_onehot",
                  "pgrad_w_mask_ignored"):
        clean = fresh_oracle("clean_pgrad")

        def pg(h, w, targets, mask, lse, g):
            h = np.asarray(h, dtype=np.float64)
            w = np.asarray(w, dtype=np.float64)
            z = h @ w.T
            d = clean.logp_backward_from_f64(z, targets, mask, lse, g)
            if name == "pgrad_sign":
                return -(d @ w), -(d.T @ h)
            if name == "pgrad_h_rows_reversed":
                return d @ w[::-1], d.T @ h
            if name == "pgrad_w_no_onehot":
                t = np.asarray(targets, dtype=np.int64)
                act = np.ones(len(t), bool) if mask is None else np.asarray(mask).astype(bool)
                d2 = d.copy()
                for i in np.nonzero(act)[0]:
                    d2[i, t[i]] -= np.asarray(g, dtype=np.float64)[i]
                return d @ w, d2.T @ h
            # mask ignored in grad_W: inactive rows with a valid target contribute
            t = np.asarray(targets, dtype=np.int64)
            tv = np.where((t < 0) | (t >= w.shape[0]), 0, t)
            d_all = clean.logp_backward_from_f64(z, tv, None, lse, g)
            return d @ w, d_all.T @ h
        o.linear_param_grads_from_f64 = pg
        o.linear_param_grads = lambda hb, wb, t, m, l, g: pg(o.bf16_to_f64(hb), o.bf16_to_f64(wb), t, m, l, g)
    else:
        raise AssertionError(name)
    return o



MUTANTS = ["sign", "no_shift", "log2", "drop_max", "mean_not_sum", "gather_off_by_one",
           "decode_as_fp16", "weight_transposed", "mask_ignored", "bwd_sign", "bwd_no_g",
           "bwd_no_onehot", "bwd_no_lse", "entropy_sign", "entropy_no_p", "log_softmax_no_lse",
           "loss_max_not_min", "loss_grad_ignores_clip", "kl_sign", "pgrad_sign",
           "pgrad_h_rows_reversed", "pgrad_w_no_onehot", "pgrad_w_mask_ignored"]


@pytest.mark.parametrize("name", MUTANTS)
def test_mutant_is_caught(name):
    o = make_mutant(name)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except Exception as e:  # AssertionError, or a crash from the bad code
            failed.append((pin.__name__, type(e).__name__))
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_copy_passes():
    o = fresh_oracle("clean")
    for pin in ALL_PINS:
        pin(o)
