"""Pins for the fp64 oracle: facts that hold independently of its code.

Each pin takes an oracle-like object ``o`` (the real ``oracle`` package, or a
deliberately broken copy in the mutant tests) and raises AssertionError when
``o`` disagrees with something fixed by mathematics rather than by the
oracle's own implementation:

* brute force on tiny vocabularies, through a separate pure-Python path
  (``math.exp`` + ``math.fsum``, no max shift);
* closed forms: uniform rows give -ln V, V = 2 gives -log1p(exp(x1 - x0)),
  one peaked entry gives -ln(1 + (V - 1) e^{-L});
* invariants: sum_t exp(logp_t) = 1, logp_t - logp_u = x_t - x_u, shift
  invariance, sum_j dlogits_ij = 0;
* special cases of the projection: one-hot hidden picks a weight column, a
  zero hidden row gives uniform logits, identical weight rows give uniform
  logits, and exact-sum spot checks of z;
* central finite differences of the forward for the backward.

The bf16 test values used here are chosen to be exactly representable, so the
pins do not depend on any rounding routine.
"""

import math

import numpy as np

# ---------------------------------------------------------------------------
# small exact bf16 helpers (test side; independent of the oracle's decoder)


def to_bf16_bits_exact(values):
    """Encode float values that are exactly representable in bf16."""
    f32 = np.asarray(values, dtype=np.float32)
    u32 = f32.view(np.uint32)
    if np.any(u32 & np.uint32(0xFFFF)):
        raise ValueError("value not exactly representable in bf16")
    return (u32 >> np.uint32(16)).astype(np.uint16)


def bf16_rne_bits(values):
    """Round float32 values to bf16 (round to nearest even), as raw bits."""
    u32 = np.asarray(values, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u32 + 0x7FFF + ((u32 >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bits_to_float(bits):
    """Test-side bf16 decode through Python floats (struct-free)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def grid_values(rng, shape, lo=-8.0, hi=8.0, step=0.125):
    """Random values on a grid that bf16 represents exactly."""
    k = rng.integers(int(lo / step), int(hi / step) + 1, size=shape)
    return k.astype(np.float64) * step


def brute_logp(row, t):
    """log softmax(row)[t] through math.exp/math.fsum, no max shift."""
    total = math.fsum(math.exp(v) for v in row)
    return row[t] - math.log(total)


# ---------------------------------------------------------------------------
# forward pins


def pin_brute_force_tiny(o):
    rng = np.random.default_rng(11)
    for v in range(1, 17):
        vals = grid_values(rng, (6, v))
        bits = to_bf16_bits_exact(vals)
        t = rng.integers(0, v, size=6)
        logp, lse = o.logp_selected(bits, t)
        for i in range(6):
            row = [float(a) for a in vals[i]]
            ref = brute_logp(row, int(t[i]))
            assert abs(logp[i] - ref) <= 1e-13, (v, i, logp[i], ref)
            ref_lse = math.log(math.fsum(math.exp(a) for a in row))
            assert abs(lse[i] - ref_lse) <= 1e-13, (v, i, lse[i], ref_lse)


def pin_uniform_rows(o):
    for v in (1, 2, 3, 1024, 32000):
        for c in (0.0, 1.5, -37.0, 1000.0, -1000.0):
            bits = to_bf16_bits_exact(np.full((2, v), c))
            t = np.array([0, v - 1])
            logp, lse = o.logp_selected(bits, t)
            tol = 8 * np.finfo(np.float64).eps * (abs(c) + math.log(v) + 1)
            assert np.all(np.abs(logp + math.log(v)) <= tol), (v, c, logp)
            assert np.all(np.abs(lse - (c + math.log(v))) <= tol), (v, c, lse)
            if v == 1:
                assert np.all(logp == 0.0), (c, logp)


def pin_uniform_large_vocab(o):
    # the two vocabularies of the workloads, through the f64 entry point
    for v in (128256, 151936):
        x = np.full((1, v), -2.5)
        logp, _ = o.selected_logp_from_f64(x, [v // 3])
        assert abs(logp[0] + math.log(v)) <= 1e-12, (v, logp)


def pin_two_entries(o):
    rng = np.random.default_rng(12)
    vals = grid_values(rng, (40, 2), -16, 16, 0.25)
    bits = to_bf16_bits_exact(vals)
    logp, _ = o.logp_selected(bits, np.zeros(40, dtype=np.int64))
    ref = -np.log1p(np.exp(vals[:, 1] - vals[:, 0]))
    assert np.max(np.abs(logp - ref)) <= 1e-14, np.max(np.abs(logp - ref))
    logp1, _ = o.logp_selected(bits, np.ones(40, dtype=np.int64))
    ref1 = -np.log1p(np.exp(vals[:, 0] - vals[:, 1]))
    assert np.max(np.abs(logp1 - ref1)) <= 1e-14


def pin_peaked_row(o):
    for v in (2, 17, 1000):
        for L in (0.5, 4.0, 20.0):
            row = np.full(v, 1.0)
            k = v // 2
            row[k] += L
            bits = to_bf16_bits_exact(row[None, :])
            logp_peak, _ = o.logp_selected(bits, [k])
            ref = -math.log1p((v - 1) * math.exp(-L))
            assert abs(logp_peak[0] - ref) <= 1e-13, (v, L, logp_peak, ref)
            other = (k + 1) % v
            logp_other, _ = o.logp_selected(bits, [other])
            assert abs(logp_other[0] - (ref - L)) <= 1e-13, (v, L)


def pin_probabilities_sum_to_one(o):
    rng = np.random.default_rng(13)
    v = 97
    vals = grid_values(rng, (1, v), -12, 12, 0.0625)
    bits = np.repeat(to_bf16_bits_exact(vals), v, axis=0)
    logp, _ = o.logp_selected(bits, np.arange(v))
    total = math.fsum(math.exp(a) for a in logp)
    assert abs(total - 1.0) <= 1e-12, total


def pin_differences_are_logit_differences(o):
    rng = np.random.default_rng(14)
    v = 300
    vals = grid_values(rng, (1, v), -20, 20, 0.25)
    bits = np.repeat(to_bf16_bits_exact(vals), 5, axis=0)
    t = rng.integers(0, v, size=5)
    logp, _ = o.logp_selected(bits, t)
    for a in range(5):
        for b in range(5):
            d = logp[a] - logp[b]
            assert abs(d - (vals[0, t[a]] - vals[0, t[b]])) <= 1e-12, (a, b)


def pin_shift_invariance(o):
    rng = np.random.default_rng(15)
    x = grid_values(rng, (4, 50), -5, 5, 0.5)
    t = rng.integers(0, 50, size=4)
    lp0, lse0 = o.selected_logp_from_f64(x, t)
    lp1, lse1 = o.selected_logp_from_f64(x + 64.0, t)
    assert np.max(np.abs(lp0 - lp1)) <= 1e-12
    assert np.max(np.abs((lse1 - lse0) - 64.0)) <= 1e-12


def pin_mask_and_targets(o):
    rng = np.random.default_rng(16)
    vals = grid_values(rng, (5, 8))
    bits = to_bf16_bits_exact(vals)
    t = np.array([1, -100, 3, 999, 0])
    mask = np.array([1, 0, 1, 0, 1], dtype=np.uint8)
    logp, lse = o.logp_selected(bits, t, mask)
    assert logp[1] == 0.0 and lse[1] == 0.0 and logp[3] == 0.0 and lse[3] == 0.0
    for i in (0, 2, 4):
        ref = brute_logp([float(a) for a in vals[i]], int(t[i]))
        assert abs(logp[i] - ref) <= 1e-13
    try:
        o.logp_selected(bits, t)  # all rows active: row 1 has target -100
    except ValueError:
        pass
    else:
        raise AssertionError("active row with an invalid target must raise")


def pin_nonfinite(o):
    ninf = -np.inf
    x = np.array([[0.0, ninf, 0.0, ninf], [ninf, ninf, ninf, ninf], [1.0, np.inf, 0.0, 0.0],
                  [np.nan, 0.0, 0.0, 0.0]])
    logp, lse = o.selected_logp_from_f64(x, [0, 0, 0, 1])
    assert abs(logp[0] + math.log(2.0)) <= 1e-15, logp[0]
    assert np.isnan(lse[1]) and np.isnan(lse[2]) and np.isnan(lse[3]), lse


# ---------------------------------------------------------------------------
# projection pins


def _rand_bf16(rng, shape, scale):
    return bf16_rne_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def pin_projection_spot_checks(o):
    rng = np.random.default_rng(21)
    n, v, h = 3, 7, 40   # non-square on purpose: a transposed operand cannot fit
    hb = _rand_bf16(rng, (n, h), 1.0)
    wb = _rand_bf16(rng, (v, h), 0.5)
    z = o.linear_logits(hb, wb)
    assert z.shape == (n, v), z.shape
    hf = bits_to_float(hb)
    wf = bits_to_float(wb)
    for i in range(n):
        for j in range(v):
            ref = math.fsum(float(hf[i, k]) * float(wf[j, k]) for k in range(h))
            assert abs(z[i, j] - ref) <= 1e-12 * (1 + abs(ref)), (i, j, z[i, j], ref)


def pin_projection_one_hot(o):
    rng = np.random.default_rng(22)
    v, h = 9, 16
    wb = _rand_bf16(rng, (v, h), 1.0)
    hid = np.zeros((h, h))
    np.fill_diagonal(hid, 1.0)
    z = o.linear_logits(to_bf16_bits_exact(hid), wb)
    assert np.array_equal(z, bits_to_float(wb).T), "one-hot hidden must pick weight columns"


def pin_projection_zero_hidden_and_equal_rows(o):
    rng = np.random.default_rng(23)
    v, h = 33, 24
    wb = _rand_bf16(rng, (v, h), 1.0)
    logp, _ = o.linear_logp(np.zeros((2, h), dtype=np.uint16), wb, [0, 5])
    assert np.max(np.abs(logp + math.log(v))) <= 1e-14
    row = _rand_bf16(rng, (1, h), 1.0)
    same = np.repeat(row, v, axis=0)
    hb = _rand_bf16(rng, (3, h), 1.0)
    logp2, _ = o.linear_logp(hb, same, [1, 2, 3])
    assert np.max(np.abs(logp2 + math.log(v))) <= 1e-12


def pin_fused_matches_brute_force(o):
    rng = np.random.default_rng(24)
    n, v, h = 4, 11, 12
    hb = _rand_bf16(rng, (n, h), 1.0)
    wb = _rand_bf16(rng, (v, h), 1.0)
    t = rng.integers(0, v, size=n)
    mask = np.array([1, 1, 0, 1], dtype=np.uint8)
    logp, _ = o.linear_logp(hb, wb, t, mask)
    hf, wf = bits_to_float(hb), bits_to_float(wb)
    for i in range(n):
        if not mask[i]:
            assert logp[i] == 0.0
            continue
        z = [math.fsum(float(hf[i, k]) * float(wf[j, k]) for k in range(h)) for j in range(v)]
        assert abs(logp[i] - brute_logp(z, int(t[i]))) <= 1e-13


# ---------------------------------------------------------------------------
# backward pins


def pin_backward_rows_sum_to_zero(o):
    rng = np.random.default_rng(31)
    x = rng.standard_normal((6, 200)) * 3
    t = rng.integers(0, 200, size=6)
    g = rng.standard_normal(6)
    _, lse = o.selected_logp_from_f64(x, t)
    d = o.logp_backward_from_f64(x, t, None, lse, g)
    assert np.all(np.abs(d.sum(axis=1)) <= 1e-12 * (1 + np.abs(g)))
    # the target entry carries g * (1 - p_t) > 0 share of the sign of g
    for i in range(6):
        assert np.sign(d[i, t[i]]) == np.sign(g[i])


def pin_backward_closed_forms(o):
    v = 10
    x = np.full((3, v), 2.0)
    t = np.array([0, 4, 9])
    g = np.array([1.5, -0.25, 0.0])
    _, lse = o.selected_logp_from_f64(x, t)
    d = o.logp_backward_from_f64(x, t, None, lse, g)
    for i in range(3):
        ref = np.full(v, -g[i] / v)
        ref[t[i]] += g[i]
        assert np.max(np.abs(d[i] - ref)) <= 1e-15, (i, d[i], ref)
    x1 = np.array([[3.0], [-7.0]])
    _, lse1 = o.selected_logp_from_f64(x1, [0, 0])
    d1 = o.logp_backward_from_f64(x1, [0, 0], None, lse1, [2.0, -1.0])
    assert np.max(np.abs(d1)) <= 1e-15, d1


def pin_backward_finite_differences(o):
    rng = np.random.default_rng(32)
    for v in (2, 5, 16):
        x = rng.standard_normal((1, v)) * 2
        t = [int(rng.integers(0, v))]
        g = float(rng.standard_normal())
        _, lse = o.selected_logp_from_f64(x, t)
        d = o.logp_backward_from_f64(x, t, None, lse, [g])
        # with no lse given the oracle takes its own: the same gradient
        d_own = o.logp_backward_from_f64(x, t, None, None, [g])
        eps = 1e-6
        for j in range(v):
            xp = x.copy()
            xm = x.copy()
            xp[0, j] += eps
            xm[0, j] -= eps
            fp = o.selected_logp_from_f64(xp, t)[0][0]
            fm = o.selected_logp_from_f64(xm, t)[0][0]
            fd = g * (fp - fm) / (2 * eps)
            assert abs(d[0, j] - fd) <= 1e-7 * (1 + abs(g)), (v, j, d[0, j], fd)
            assert abs(d_own[0, j] - fd) <= 1e-7 * (1 + abs(g)), (v, j, d_own[0, j], fd)


def pin_backward_mask(o):
    rng = np.random.default_rng(33)
    vals = grid_values(rng, (3, 6))
    bits = to_bf16_bits_exact(vals)
    t = np.array([2, -100, 5])
    mask = np.array([1, 0, 1], dtype=np.uint8)
    _, lse = o.logp_selected(bits, t, mask)
    d = o.logp_backward(bits, t, mask, lse, [1.0, 3.0, -2.0])
    assert np.all(d[1] == 0.0)
    row = [float(a) for a in vals[0]]
    tot = math.fsum(math.exp(a) for a in row)
    for j in range(6):
        ref = (1.0 if j == 2 else 0.0) - math.exp(row[j]) / tot
        assert abs(d[0, j] - ref) <= 1e-14


def pin_linear_backward_matches_brute_force(o):
    rng = np.random.default_rng(34)
    n, v, h = 3, 7, 10
    hb = _rand_bf16(rng, (n, h), 1.0)
    wb = _rand_bf16(rng, (v, h), 1.0)
    t = rng.integers(0, v, size=n)
    g = rng.standard_normal(n)
    _, lse = o.linear_logp(hb, wb, t)
    d = o.linear_logp_backward(hb, wb, t, None, lse, g)
    hf, wf = bits_to_float(hb), bits_to_float(wb)
    for i in range(n):
        z = [math.fsum(float(hf[i, k]) * float(wf[j, k]) for k in range(h)) for j in range(v)]
        tot = math.fsum(math.exp(a) for a in z)
        for j in range(v):
            ref = g[i] * ((1.0 if j == t[i] else 0.0) - math.exp(z[j]) / tot)
            assert abs(d[i, j] - ref) <= 1e-13, (i, j)


ALL_PINS = [
    pin_brute_force_tiny,
    pin_uniform_rows,
    pin_uniform_large_vocab,
    pin_two_entries,
    pin_peaked_row,
    pin_probabilities_sum_to_one,
    pin_differences_are_logit_differences,
    pin_shift_invariance,
    pin_mask_and_targets,
    pin_nonfinite,
    pin_projection_spot_checks,
    pin_projection_one_hot,
    pin_projection_zero_hidden_and_equal_rows,
    pin_fused_matches_brute_force,
    pin_backward_rows_sum_to_zero,
    pin_backward_closed_forms,
    pin_backward_finite_differences,
    pin_backward_mask,
    pin_linear_backward_matches_brute_force,
]


# ---------------------------------------------------------------------------
# dense log-softmax and entropy pins


def pin_entropy_brute_force(o):
    rng = np.random.default_rng(41)
    for v in range(1, 13):
        vals = grid_values(rng, (4, v))
        h = o.entropy(to_bf16_bits_exact(vals))
        for i in range(4):
            row = [float(a) for a in vals[i]]
            tot = math.fsum(math.exp(a) for a in row)
            ps = [math.exp(a) / tot for a in row]
            ref = -math.fsum(p * math.log(p) for p in ps if p > 0)
            assert abs(h[i] - ref) <= 1e-13, (v, i, h[i], ref)


def pin_entropy_closed_forms(o):
    for v in (1, 2, 1000, 151936):
        h = o.entropy_from_f64(np.full((1, v), 3.25))
        assert abs(h[0] - math.log(v)) <= 1e-12, (v, h)
    # two entries: binary entropy of sigmoid(x0 - x1)
    rng = np.random.default_rng(42)
    x = rng.standard_normal((20, 2)) * 4
    h = o.entropy_from_f64(x)
    p = 1.0 / (1.0 + np.exp(x[:, 1] - x[:, 0]))
    ref = -(p * np.log(p) + (1 - p) * np.log1p(-p))
    assert np.max(np.abs(h - ref)) <= 1e-12
    # -inf entries contribute nothing: [0, -inf, 0] has entropy ln 2
    h2 = o.entropy_from_f64(np.array([[0.0, -np.inf, 0.0]]))
    assert abs(h2[0] - math.log(2.0)) <= 1e-15
    # masked rows are zero
    h3 = o.entropy_from_f64(np.ones((2, 5)), np.array([0, 1], dtype=np.uint8))
    assert h3[0] == 0.0 and abs(h3[1] - math.log(5)) <= 1e-15


def pin_entropy_bounds(o):
    rng = np.random.default_rng(43)
    x = rng.standard_normal((50, 300)) * rng.uniform(0.1, 20, size=(50, 1))
    h = o.entropy_from_f64(x)
    assert np.all(h >= -1e-12) and np.all(h <= math.log(300) + 1e-12)
    # sharper rows have lower entropy (scaling the logits up by 2)
    h2 = o.entropy_from_f64(2 * x)
    assert np.all(h2 <= h + 1e-12)


def pin_log_softmax_rows(o):
    rng = np.random.default_rng(44)
    vals = grid_values(rng, (3, 40), -10, 10, 0.25)
    ls = o.log_softmax(to_bf16_bits_exact(vals), np.array([1, 0, 1], dtype=np.uint8))
    assert np.all(ls[1] == 0.0)
    for i in (0, 2):
        row = [float(a) for a in vals[i]]
        lse = math.log(math.fsum(math.exp(a) for a in row))
        assert np.max(np.abs(ls[i] - (vals[i] - lse))) <= 1e-13
        assert abs(math.fsum(math.exp(a) for a in ls[i]) - 1.0) <= 1e-13
    u = o.log_softmax_from_f64(np.full((1, 64), -7.0))
    assert np.max(np.abs(u + math.log(64))) <= 1e-15


ALL_PINS += [pin_entropy_brute_force, pin_entropy_closed_forms, pin_entropy_bounds,
             pin_log_softmax_rows]


# ---------------------------------------------------------------------------
# per-token loss pins


def pin_token_losses_closed_forms(o):
    # on-policy (logp == logp_old): ratio 1, surrogate -A, gradient -A
    rng = np.random.default_rng(51)
    lp = rng.standard_normal(64) * 3 - 5
    a = rng.standard_normal(64)
    out = o.token_losses(lp, lp, a)
    assert np.all(out["ratio"] == 1.0)
    assert np.max(np.abs(out["loss"] + a)) <= 1e-15
    assert np.max(np.abs(out["grad"] + a)) <= 1e-15
    # clipping: with A > 0 and ratio above 1 + eps the loss is -(1+eps) A
    # and the gradient 0; with A < 0 and ratio below 1 - eps the loss is
    # -(1-eps) A and the gradient 0
    out2 = o.token_losses(np.array([0.5, -0.5]), np.array([0.0, 0.0]), np.array([2.0, -3.0]),
                          eps_lo=0.1, eps_hi=0.3)
    assert abs(out2["loss"][0] + 1.3 * 2.0) <= 1e-15 and out2["grad"][0] == 0.0
    assert abs(out2["loss"][1] + 0.9 * -3.0) <= 1e-15 and out2["grad"][1] == 0.0
    # A > 0 with ratio below 1 - eps is not clipped: loss -ratio A
    out3 = o.token_losses(np.array([-1.0]), np.array([0.0]), np.array([1.5]), eps_lo=0.2)
    r = math.exp(-1.0)
    assert abs(out3["loss"][0] + r * 1.5) <= 1e-15 and abs(out3["grad"][0] + r * 1.5) <= 1e-15
    # masked tokens are zero
    out4 = o.token_losses(lp[:3], lp[:3] + 1, a[:3], np.array([1, 0, 1], dtype=np.uint8))
    for k in ("ratio", "loss", "kl", "grad"):
        assert out4[k][1] == 0.0


def pin_token_kl(o):
    rng = np.random.default_rng(52)
    lp = rng.standard_normal(200) * 2 - 4
    ref = lp + rng.standard_normal(200)
    out = o.token_losses(lp, lp, np.zeros(200), logp_ref=ref, beta=0.5)
    d = ref - lp
    assert np.all(out["kl"] >= -1e-15)                       # e^d - d - 1 >= 0
    assert np.max(np.abs(out["kl"] - (np.expm1(d) - d))) <= 1e-12
    same = o.token_losses(lp, lp, np.zeros(200), logp_ref=lp, beta=0.5)
    assert np.all(same["kl"] == 0.0) and np.all(same["grad"] == 0.0)
    # small-difference expansion kl ~ d^2 / 2
    tiny = o.token_losses(np.array([0.0]), np.array([0.0]), np.array([0.0]),
                          logp_ref=np.array([1e-3]), beta=1.0)
    assert abs(tiny["kl"][0] - 0.5e-6) <= 1e-9


def pin_token_loss_gradient_fd(o):
    rng = np.random.default_rng(53)
    lp = rng.standard_normal(40) * 0.5 - 3
    old = lp + rng.standard_normal(40) * 0.4
    ref = lp + rng.standard_normal(40) * 0.3
    a = rng.standard_normal(40)
    kw = dict(logp_ref=ref, eps_lo=0.2, eps_hi=0.28, beta=0.04)
    g = o.token_losses(lp, old, a, **kw)["grad"]
    h = 1e-6
    fp = o.token_losses(lp + h, old, a, **kw)["loss"]
    fm = o.token_losses(lp - h, old, a, **kw)["loss"]
    fd = (fp - fm) / (2 * h)
    r = np.exp(lp - old)
    near_edge = (np.abs(r - 0.8) < 1e-4) | (np.abs(r - 1.28) < 1e-4)
    assert np.max(np.abs((g - fd)[~near_edge])) <= 1e-6


ALL_PINS += [pin_token_losses_closed_forms, pin_token_kl, pin_token_loss_gradient_fd]


# ---------------------------------------------------------------------------
# parameter-gradient pins (grad_hidden = D . W, grad_weight = D^T . h)


def _brute_loss(hf, wf, t, g, act):
    """sum_i g_i logp_i over active rows, through math.fsum/math.exp only."""
    n, hh = hf.shape
    v = wf.shape[0]
    total = []
    for i in range(n):
        if not act[i]:
            continue
        z = [math.fsum(float(hf[i, k]) * float(wf[j, k]) for k in range(hh)) for j in range(v)]
        total.append(float(g[i]) * brute_logp(z, int(t[i])))
    return math.fsum(total)


def pin_param_grads_finite_differences(o):
    rng = np.random.default_rng(41)
    n, v, hh = 3, 5, 4          # all different, so a transposed operand cannot fit
    hf = rng.standard_normal((n, hh))
    wf = rng.standard_normal((v, hh)) * 0.7
    t = np.array([1, 4, 0])
    g = rng.standard_normal(n)
    act = np.array([True, False, True])
    mask = act.astype(np.uint8)
    lse = np.zeros(n)
    for i in range(n):
        z = [math.fsum(float(hf[i, k]) * float(wf[j, k]) for k in range(hh)) for j in range(v)]
        lse[i] = math.log(math.fsum(math.exp(a) for a in z))
    gh, gw = o.linear_param_grads_from_f64(hf, wf, t, mask, lse, g)
    assert gh.shape == (n, hh) and gw.shape == (v, hh), (gh.shape, gw.shape)
    # with no lse given the oracle takes its own from the same h and W
    gh_own, gw_own = o.linear_param_grads_from_f64(hf, wf, t, mask, None, g)
    eps = 1e-6
    for arr, grad in ((hf, gh), (wf, gw), (hf, gh_own), (wf, gw_own)):
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + eps
            fp = _brute_loss(hf, wf, t, g, act)
            arr[idx] = keep - eps
            fm = _brute_loss(hf, wf, t, g, act)
            arr[idx] = keep
            fd = (fp - fm) / (2 * eps)
            assert abs(grad[idx] - fd) <= 1e-7 * (1 + abs(fd)), (idx, grad[idx], fd)
    assert np.all(gh[1] == 0.0), "inactive row must get a zero hidden gradient"


def pin_param_grads_closed_forms(o):
    rng = np.random.default_rng(42)
    v, hh = 6, 5
    w = rng.standard_normal((v, hh))
    # zero hidden rows: z = 0, p = 1/V, so grad_h_i = g_i (W[t_i] - mean_j W_j)
    # and grad_W = 0 (every product carries a factor h = 0)
    t = np.array([2, 5])
    g = np.array([1.25, -0.5])
    h0 = np.zeros((2, hh))
    lse0 = np.full(2, math.log(v))
    gh, gw = o.linear_param_grads_from_f64(h0, w, t, None, lse0, g)
    for i in range(2):
        ref = g[i] * (w[t[i]] - w.mean(axis=0))
        assert np.max(np.abs(gh[i] - ref)) <= 1e-14, (i, gh[i], ref)
    assert np.max(np.abs(gw)) == 0.0
    # identical weight rows: logits uniform again; grad_h = g_i (w - w) = 0 and
    # grad_W_j = sum_i g_i ([j == t_i] - 1/V) h_i
    same = np.repeat(rng.standard_normal((1, hh)), v, axis=0)
    h = rng.standard_normal((3, hh))
    t3 = np.array([0, 3, 3])
    g3 = np.array([0.5, 2.0, -1.0])
    lse3 = (h @ same[0]) + math.log(v)
    gh3, gw3 = o.linear_param_grads_from_f64(h, same, t3, None, lse3, g3)
    assert np.max(np.abs(gh3)) <= 1e-14, gh3
    for j in range(v):
        ref = sum(g3[i] * ((1.0 if j == t3[i] else 0.0) - 1.0 / v) * h[i] for i in range(3))
        assert np.max(np.abs(gw3[j] - ref)) <= 1e-14, (j, gw3[j], ref)


def pin_param_grads_invariants(o):
    rng = np.random.default_rng(43)
    n, v, hh = 7, 19, 12
    hb = _rand_bf16(rng, (n, hh), 1.0)
    wb = _rand_bf16(rng, (v, hh), 0.5)
    t = rng.integers(0, v, size=n)
    g = rng.standard_normal(n)
    mask = np.array([1, 0, 1, 1, 0, 1, 1], dtype=np.uint8)
    t[1] = -100           # inactive rows may hold invalid targets
    _, lse = o.linear_logp(hb, wb, t, mask)
    gh, gw = o.linear_param_grads(hb, wb, t, mask, lse, g)
    # every row of D sums to zero, so the rows of grad_W sum to zero
    assert np.max(np.abs(gw.sum(axis=0))) <= 1e-12
    # inactive rows: zero hidden gradient, and no share in grad_W: the result
    # equals the one over the compacted active rows alone
    assert np.all(gh[mask == 0] == 0.0)
    keep = np.nonzero(mask)[0]
    gh_c, gw_c = o.linear_param_grads(hb[keep], wb, t[keep], None, lse[keep], g[keep])
    assert np.max(np.abs(gh_c - gh[keep])) <= 1e-13
    assert np.max(np.abs(gw_c - gw)) <= 1e-13
    # what an inactive row holds does not matter, NaN and infinities included
    # (grad_W is a sum over the active tokens)
    hp = hb.copy()
    hp[1, :] = 0x7FC0                 # NaN
    hp[4, ::2] = 0x7F80               # +inf
    hp[4, 1::2] = 0xFF80              # -inf
    with np.errstate(invalid="ignore", over="ignore"):   # the poisoned rows' own logits
        gh_p, gw_p = o.linear_param_grads(hp, wb, t, mask, lse, g)
        vr = [int(t[0]), 3, v - 1]
        gw_r = o.linear_grad_weight_rows(hp, wb, t, mask, lse, g, vr)
    assert np.all(np.isfinite(gw_p)) and np.array_equal(gw_p, gw)
    assert np.array_equal(gh_p, gh)
    assert np.array_equal(gw_r, gw[vr])


ALL_PINS += [pin_param_grads_finite_differences, pin_param_grads_closed_forms,
             pin_param_grads_invariants]


def pin_param_grad_row_samplers(o):
    """The per-row samplers used at full sizes agree with the full
    (finite-difference pinned) parameter gradients."""
    rng = np.random.default_rng(44)
    n, v, hh = 9, 70, 16
    hb = _rand_bf16(rng, (n, hh), 1.0)
    wb = _rand_bf16(rng, (v, hh), 0.5)
    t = rng.integers(0, v, size=n)
    g = rng.standard_normal(n)
    mask = np.ones(n, dtype=np.uint8)
    mask[[2, 7]] = 0
    _, lse = o.linear_logp(hb, wb, t, mask)
    gh, gw = o.linear_param_grads(hb, wb, t, mask, lse, g)
    rows = [0, 2, 8]
    gh_s = o.linear_grad_hidden_rows(hb, wb, t, mask, lse, g, rows, block=16)
    assert np.max(np.abs(gh_s - gh[rows])) <= 1e-13
    vr = [int(t[0]), 5, v - 1]
    gw_s = o.linear_grad_weight_rows(hb, wb, t, mask, lse, g, vr)
    assert np.max(np.abs(gw_s - gw[vr])) <= 1e-13
    # with no lse given, the samplers take the oracle's own
    gh_o = o.linear_grad_hidden_rows(hb, wb, t, mask, None, g, rows, block=16)
    gw_o = o.linear_grad_weight_rows(hb, wb, t, mask, None, g, vr)
    assert np.max(np.abs(gh_o - gh[rows])) <= 1e-13
    assert np.max(np.abs(gw_o - gw[vr])) <= 1e-13


ALL_PINS += [pin_param_grad_row_samplers]
