"""Plain fp64 CPU oracle for the batch-invariant selected-token log-probability.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code, header, table or helper with the
HIP library; the two meet only at the seeded inputs.

What it computes, and where it comes from
-----------------------------------------
The pages name the operator -- "selected logprob" / ``logp`` /
``batch_invariant_logp`` and the fused ``linear_logp`` (page "docs(ws1):
batch-invariance contract RFC", section "First-Divergence Localization", the
operator chain, entries 6-8; page "[RFC] Batch-Invariant RL Kernel Suite for
Train-Inference Consistency", section "Scope", dense vs indexed
selected-logprob paths) -- but never write its formula.  The oracle therefore
uses the textbook definition: for a row of logits ``x`` and a target index
``t``

    lse(x)  = log( sum_j exp(x_j) )
    logp    = x_t - lse(x)
    dlogp/dx_j = [j == t] - exp(x_j - lse(x))          (backward, times g)

Inputs are bf16 (page "[WS1 Test] #154 dtype pin + ...", section "Workstream
1 - #154 dtype coverage", scope table: BF16 inputs, FP32 accumulation, FP32
gold).  This oracle is stricter than an fp32 gold: every bf16 value is decoded
exactly and all arithmetic is float64.

Masked (inactive) rows are excluded from comparisons (page "docs(ws1): ...",
section "InvarianceFixture", requirement 3; page "[WS1 Test] ...", section
"Workstream 3 - #153", logical-workload identity: padding tokens are
excluded); the oracle reports zeros for them, which is also what the library
writes.

Parity is pinned by ``tests/oracle_pins.py`` (brute force on tiny vocabularies,
closed forms, invariants, finite differences); every function here has pins.
"""

import numpy as np

LN2 = float(np.log(2.0))


def bf16_to_f64(bits):
    """Exact bf16 -> float64 decode of raw 16-bit patterns.

    A bf16 value is the upper half of an IEEE float32, so shifting the 16 bits
    into the high half of a 32-bit word and reinterpreting it is exact.
    """
    u16 = np.ascontiguousarray(bits, dtype=np.uint16)
    u32 = u16.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def _active(mask, n):
    if mask is None:
        return np.ones(n, dtype=bool)
    return np.asarray(mask).astype(bool).reshape(n)


def logsumexp_rows(x):
    """Row-wise natural-log sum of exponentials of a float64 matrix.

    The maximum is subtracted before exponentiating (the usual overflow-safe
    rewriting; mathematically identical).  -inf entries contribute nothing;
    a row containing +inf or NaN yields NaN; an all -inf row yields NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=1)
    out = np.full(x.shape[0], np.nan)
    ok = np.isfinite(m) & ~np.isnan(x).any(axis=1)
    if ok.any():
        xs = x[ok]
        mm = m[ok]
        with np.errstate(invalid="ignore", over="ignore"):
            s = np.sum(np.exp(xs - mm[:, None]), axis=1)
        out[ok] = mm + np.log(s)
    return out


def selected_logp_from_f64(x, targets, mask=None):
    """logp and lse for float64 logits ``x`` [N, V].

    Returns (logp, lse) as float64 [N].  Inactive rows give 0 for both.  An
    active row whose target is outside [0, V) is an error.
    """
    x = np.asarray(x, dtype=np.float64)
    n, v = x.shape
    t = np.asarray(targets, dtype=np.int64).reshape(n)
    act = _active(mask, n)
    logp = np.zeros(n)
    lse = np.zeros(n)
    if not act.any():
        return logp, lse
    if np.any((t[act] < 0) | (t[act] >= v)):
        raise ValueError("active row with target outside [0, V)")
    rows = np.nonzero(act)[0]
    lse_a = logsumexp_rows(x[rows])
    lse[rows] = lse_a
    logp[rows] = x[rows, t[rows]] - lse_a
    return logp, lse


def logp_selected(logits_bits, targets, mask=None, block_rows=256):
    """Selected-token logprob from bf16 logits given as raw uint16 [N, V].

    Rows are processed in blocks only to bound host memory.
    """
    bits = np.asarray(logits_bits, dtype=np.uint16)
    n, v = bits.shape
    t = np.asarray(targets, dtype=np.int64).reshape(n)
    act = _active(mask, n)
    logp = np.zeros(n)
    lse = np.zeros(n)
    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        lp, ls = selected_logp_from_f64(bf16_to_f64(bits[r0:r1]), t[r0:r1], act[r0:r1])
        logp[r0:r1] = lp
        lse[r0:r1] = ls
    return logp, lse


def linear_logits(hidden_bits, weight_bits):
    """Logits of the lm_head projection, z = h . W^T, in float64.

    ``hidden_bits`` is bf16 [N, H], ``weight_bits`` is bf16 [V, H] (the
    nn.Linear weight layout: one row per vocabulary entry, H contiguous).
    Each bf16 x bf16 product is exact in float64; the sum is a float64 BLAS
    dot product.
    """
    h = bf16_to_f64(hidden_bits)
    w = bf16_to_f64(weight_bits)
    if h.shape[1] != w.shape[1]:
        raise ValueError("hidden and weight disagree on H")
    return h @ w.T


def linear_logp(hidden_bits, weight_bits, targets, mask=None, block_rows=256):
    """Fused lm_head + selected logprob: (logp, lse) float64 [N].

    The logits are never rounded: they stay float64 here (the library keeps
    them float32 and never rounds them to bf16).
    """
    h = np.asarray(hidden_bits, dtype=np.uint16)
    w = bf16_to_f64(weight_bits)
    n = h.shape[0]
    t = np.asarray(targets, dtype=np.int64).reshape(n)
    act = _active(mask, n)
    logp = np.zeros(n)
    lse = np.zeros(n)
    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        z = bf16_to_f64(h[r0:r1]) @ w.T
        lp, ls = selected_logp_from_f64(z, t[r0:r1], act[r0:r1])
        logp[r0:r1] = lp
        lse[r0:r1] = ls
    return logp, lse


def logp_backward_from_f64(x, targets, mask, lse, grad_logp):
    """Gradient of g_i * logp_i with respect to the logits row x_i.

    d[i, j] = g_i * ([j == t_i] - exp(x_ij - lse_i)) for active rows, and 0
    for inactive rows (page "[WS1 Test] ...", section "Workstream 3 - #153":
    padding is excluded and the upstream gradients are identical across
    configurations; the formula itself is the textbook derivative of the
    definition above).

    ``lse`` is the log-sum-exp of each row.  ``None`` means the oracle's own,
    computed here from the same logits: the gradient of the whole definition,
    from the inputs alone (the end-to-end reference).  A given array makes
    this the backward as a function of that lse.
    """
    x = np.asarray(x, dtype=np.float64)
    n, v = x.shape
    t = np.asarray(targets, dtype=np.int64).reshape(n)
    act = _active(mask, n)
    g = np.asarray(grad_logp, dtype=np.float64).reshape(n)
    if lse is None:
        ls = np.zeros(n)
        rows_a = np.nonzero(act)[0]
        if rows_a.size:
            ls[rows_a] = logsumexp_rows(x[rows_a])
    else:
        ls = np.asarray(lse, dtype=np.float64).reshape(n)
    d = np.zeros((n, v))
    rows = np.nonzero(act)[0]
    if rows.size:
        if np.any((t[rows] < 0) | (t[rows] >= v)):
            raise ValueError("active row with target outside [0, V)")
        p = np.exp(x[rows] - ls[rows, None])
        onehot = np.zeros((rows.size, v))
        onehot[np.arange(rows.size), t[rows]] = 1.0
        d[rows] = g[rows, None] * (onehot - p)
    return d


def logp_backward(logits_bits, targets, mask, lse, grad_logp):
    """Backward from bf16 logits (raw uint16 [N, V]); float64 [N, V].
    ``lse`` None: the oracle's own (see logp_backward_from_f64)."""
    return logp_backward_from_f64(bf16_to_f64(logits_bits), targets, mask, lse, grad_logp)


def linear_logp_backward(hidden_bits, weight_bits, targets, mask, lse, grad_logp):
    """Backward of the fused path with respect to the (never materialised)
    logits z = h . W^T; float64 [N, V].  ``lse`` None: the oracle's own."""
    z = linear_logits(hidden_bits, weight_bits)
    return logp_backward_from_f64(z, targets, mask, lse, grad_logp)


# ---------------------------------------------------------------------------
# Dense outputs from the same log-sum-exp: the full log-softmax row and the
# per-row entropy.  The pages contrast dense and indexed selected-logprob
# paths (page "[RFC] Batch-Invariant RL Kernel Suite for Train-Inference
# Consistency", section "Scope"); the dense path computes every
# log-probability of the row, x_j - lse.  The entropy is the textbook
# H = -sum_j p_j log p_j with p_j = exp(x_j - lse), i.e. lse - sum_j p_j x_j,
# where entries with p_j = 0 (x_j = -inf) contribute nothing.


def log_softmax_from_f64(x, mask=None):
    """Dense log-softmax rows x_j - lse (float64 [N, V]); inactive rows 0."""
    x = np.asarray(x, dtype=np.float64)
    n, v = x.shape
    act = _active(mask, n)
    out = np.zeros((n, v))
    rows = np.nonzero(act)[0]
    if rows.size:
        lse = logsumexp_rows(x[rows])
        with np.errstate(invalid="ignore"):
            out[rows] = x[rows] - lse[:, None]
    return out


def log_softmax(logits_bits, mask=None):
    return log_softmax_from_f64(bf16_to_f64(logits_bits), mask)


def entropy_from_f64(x, mask=None):
    """Per-row entropy -sum_j p_j log p_j (float64 [N]); inactive rows 0."""
    x = np.asarray(x, dtype=np.float64)
    n, v = x.shape
    act = _active(mask, n)
    ent = np.zeros(n)
    rows = np.nonzero(act)[0]
    if rows.size:
        xs = x[rows]
        lse = logsumexp_rows(xs)
        with np.errstate(invalid="ignore", over="ignore"):
            logp = xs - lse[:, None]
            p = np.exp(logp)
            terms = np.where(p > 0, p * logp, 0.0)
        h = -np.sum(terms, axis=1)
        h[~np.isfinite(lse)] = np.nan
        ent[rows] = h
    return ent


def entropy(logits_bits, mask=None, block_rows=256):
    bits = np.asarray(logits_bits, dtype=np.uint16)
    n = bits.shape[0]
    act = _active(mask, n)
    out = np.zeros(n)
    for r0 in range(0, n, block_rows):
        r1 = min(n, r0 + block_rows)
        out[r0:r1] = entropy_from_f64(bf16_to_f64(bits[r0:r1]), act[r0:r1])
    return out


# ---------------------------------------------------------------------------
# Per-token loss consumers of the selected logprob.  The pages place the loss
# reductions (grpo_loss, ratio_kl) at the end of the operator chain and ask,
# for bitwise invariance, that they be per-token outputs rather than batch
# reductions (page "docs(ws1): batch-invariance contract RFC", section
# "First-Divergence Localization", the review of the chain's last entry).
# They do not write the formulas; the textbook GRPO/PPO terms are used:
#
#   ratio_i = exp(logp_i - logp_old_i)
#   surr_i  = -min(ratio_i * A_i, clip(ratio_i, 1 - eps_lo, 1 + eps_hi) * A_i)
#   kl_i    = exp(ref_i - logp_i) - (ref_i - logp_i) - 1        (k3 estimator)
#   loss_i  = surr_i + beta * kl_i
#   grad_i  = d loss_i / d logp_i
#
# The clipped branch has zero gradient where it is the one min() selects.


def token_losses(logp, logp_old, adv, mask=None, logp_ref=None, eps_lo=0.2, eps_hi=0.2,
                 beta=0.0):
    """Per-token ratio, loss, kl and d loss / d logp (float64 [N] each);
    masked tokens give 0 for every output."""
    lp = np.asarray(logp, dtype=np.float64)
    old = np.asarray(logp_old, dtype=np.float64)
    a = np.asarray(adv, dtype=np.float64)
    n = lp.shape[0]
    act = _active(mask, n)
    ratio = np.exp(lp - old)
    clipped = np.clip(ratio, 1.0 - eps_lo, 1.0 + eps_hi)
    unclipped_term = ratio * a
    clipped_term = clipped * a
    surr = -np.minimum(unclipped_term, clipped_term)
    # the unclipped branch is the active one (ties included) unless the
    # clipped term is strictly smaller
    use_unclipped = unclipped_term <= clipped_term
    grad = np.where(use_unclipped, -a * ratio, 0.0)
    if logp_ref is not None:
        d = np.asarray(logp_ref, dtype=np.float64) - lp
        kl = np.exp(d) - d - 1.0
        grad = grad + beta * (1.0 - np.exp(d))
    else:
        kl = np.zeros(n)
    loss = surr + beta * kl
    out = {"ratio": ratio, "loss": loss, "kl": kl, "grad": grad}
    for k in out:
        out[k] = np.where(act, out[k], 0.0)
    return out


# ---------------------------------------------------------------------------
# Parameter gradients of the fused path.  With D the logits gradient above
# (D_ij = g_i ([j == t_i] - p_ij), zero rows for inactive tokens) and
# z = h . W^T, the chain rule gives
#
#   grad_hidden = D . W        [N, H]   (row i depends on row i of D only)
#   grad_weight = D^T . h      [V, H]   (a sum over every active token)
#
# The pages ask for gradient batch invariance and say that parameter
# gradients are compared only over the same complete set of samples (page
# "[WS1 Test] #154 dtype pin + #152 KV path + #153 bwd invariance + #150
# chain gate", section "Workstream 3 - #153", scope and logical-workload
# identity); the formulas are the textbook derivatives of the definition.


def linear_param_grads_from_f64(h, w, targets, mask, lse, grad_logp):
    """(grad_hidden [N, H], grad_weight [V, H]) float64 for float64 h, W.

    ``lse`` is the forward's log-sum-exp per row (an input of the backward,
    as for the logits gradient); None means the oracle's own from the same
    h and W (the end-to-end reference)."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if h.shape[1] != w.shape[1]:
        raise ValueError("hidden and weight disagree on H")
    d = logp_backward_from_f64(h @ w.T, targets, mask, lse, grad_logp)
    # grad_weight sums over the active tokens only: an inactive row's D is
    # zero, and leaving its hidden row out keeps whatever that row holds
    # (non-finite padding included) out of the sum
    act = _active(mask, h.shape[0])
    return d @ w, d[act].T @ h[act]


def linear_param_grads(hidden_bits, weight_bits, targets, mask, lse, grad_logp):
    """Parameter gradients from bf16 hidden [N, H] and weight [V, H] bits."""
    return linear_param_grads_from_f64(bf16_to_f64(hidden_bits), bf16_to_f64(weight_bits),
                                       targets, mask, lse, grad_logp)


def linear_grad_hidden_rows(hidden_bits, weight_bits, targets, mask, lse, grad_logp, rows,
                            block=16384):
    """Rows ``rows`` of grad_hidden = D . W (float64 [len(rows), H]).

    The same formula as linear_param_grads for a few token rows of a large
    problem; the weight is visited in blocks of vocabulary rows only to bound
    host memory.  ``lse`` None: the oracle's own, for these rows."""
    hb = np.asarray(hidden_bits, dtype=np.uint16)
    wb = np.asarray(weight_bits, dtype=np.uint16)
    n = hb.shape[0]
    v, hh = wb.shape
    t = np.asarray(targets, dtype=np.int64).reshape(n)
    act = _active(mask, n)
    g = np.asarray(grad_logp, dtype=np.float64).reshape(n)
    rows = [int(r) for r in rows]
    if lse is None:
        ls = np.zeros(n)
        sel = np.asarray(rows, dtype=np.int64)
        _, ls_rows = linear_logp(hb[sel], wb, t[sel], act[sel])
        ls[sel] = ls_rows
    else:
        ls = np.asarray(lse, dtype=np.float64).reshape(n)
    out = np.zeros((len(rows), hh))
    h = bf16_to_f64(hb[rows])
    for k0 in range(0, v, block):
        k1 = min(v, k0 + block)
        w = bf16_to_f64(wb[k0:k1])
        z = h @ w.T
        for a, i in enumerate(rows):
            if not act[i]:
                continue
            if not (0 <= t[i] < v):
                raise ValueError("active row with target outside [0, V)")
            d = -g[i] * np.exp(z[a] - ls[i])
            if k0 <= t[i] < k1:
                d[t[i] - k0] += g[i]
            out[a] += d @ w
    return out


def linear_grad_weight_rows(hidden_bits, weight_bits, targets, mask, lse, grad_logp, vocab_rows):
    """Rows ``vocab_rows`` of grad_weight = D^T . h (float64 [len, H]): the
    same formula as linear_param_grads for a few vocabulary rows.  ``lse``
    None: the oracle's own (a full forward over every row)."""
    hb = np.asarray(hidden_bits, dtype=np.uint16)
    n = hb.shape[0]
    t = np.asarray(targets, dtype=np.int64).reshape(n)
    act = _active(mask, n)
    g = np.asarray(grad_logp, dtype=np.float64).reshape(n)
    if lse is None:
        _, ls = linear_logp(hb, weight_bits, t, act)
    else:
        ls = np.asarray(lse, dtype=np.float64).reshape(n)
    vocab_rows = np.asarray(vocab_rows, dtype=np.int64)
    h = bf16_to_f64(hb)
    w = bf16_to_f64(np.asarray(weight_bits, dtype=np.uint16)[vocab_rows])
    z = h @ w.T                                   # [N, k]
    d = np.zeros_like(z)
    rows = np.nonzero(act)[0]
    d[rows] = -g[rows, None] * np.exp(z[rows] - ls[rows, None])
    for i in rows:
        d[i, vocab_rows == t[i]] += g[i]
    return d[rows].T @ h[rows]
