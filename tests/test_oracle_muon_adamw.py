"""Pins for the oracle's Muon and AdamW (CPU only).

* momentum: closed form of the heavy-ball recursion;
* Newton-Schulz: the spectral closed form U p^5(S) V^T from LAPACK's SVD,
  where p(s) = a s + b s^3 + c s^5, on wide, tall and square inputs; plus the
  special cases (zero, orthonormal rows, diagonal input, scale invariance,
  orthogonal equivariance, transpose);
* AdamW: closed forms from a zero state and under a constant gradient.
A mistake planted in the oracle (sign of a coefficient, a transposed
operand, a dropped bias correction) is shown to fail these pins.
"""

import numpy as np
import pytest

import oracle

A, B, C = 3.4445, -4.7750, 2.0315
F32 = lambda x: float(np.float32(x))


def _p5(s, a=F32(A), b=F32(B), c=F32(C), steps=5):
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def _spectral(u, eps=F32(1e-7)):
    u = np.asarray(u, dtype=np.float64)
    x0 = u / (np.linalg.norm(u) + eps)
    U, S, Vt = np.linalg.svd(x0, full_matrices=False)
    return (U * _p5(S)) @ Vt


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ----------------------------------------------------------------- momentum
def test_momentum_closed_form_constant_grad():
    rng = np.random.default_rng(0)
    g = (rng.standard_normal((8, 16)) * 1e-3).astype(np.float32)
    m = np.zeros_like(g)
    mu = 0.95
    for t in range(1, 21):
        m, u = oracle.momentum_step(m, g, mu)
        ref = g.astype(np.float64) * (1 - F32(mu) ** t) / (1 - F32(mu))
        assert np.max(np.abs(m - ref) / np.abs(ref)) < 2e-6
    assert np.array_equal(u, oracle.bf16_rne(m))


def test_momentum_sum_form_varying_grad():
    rng = np.random.default_rng(1)
    gs = [(rng.standard_normal(64) * 1e-3).astype(np.float32) for _ in range(6)]
    m = np.zeros(64, np.float32)
    for g in gs:
        m, _ = oracle.momentum_step(m, g, 0.9)
    mu = F32(0.9)
    ref = sum(mu ** (len(gs) - 1 - k) * gs[k].astype(np.float64) for k in range(len(gs)))
    assert np.max(np.abs(m - ref)) < 1e-8


def test_nesterov_form():
    g = np.array([1.0, -2.0], np.float32)
    m = np.array([0.5, 0.25], np.float32)
    m_new, u = oracle.momentum_step(m, g, 0.5, nesterov=True)
    assert np.allclose(m_new, [1.25, -1.875])
    assert np.allclose(u, oracle.bf16_rne(np.float32([1.0 + 0.625, -2.0 - 0.9375])))


# ----------------------------------------------------------------- Newton-Schulz
@pytest.mark.parametrize("shape", [(16, 40), (40, 16), (24, 24), (1, 8), (64, 256), (5, 3)])
def test_ns_matches_spectral_closed_form(shape):
    rng = np.random.default_rng(hash(shape) % 2 ** 32)
    u = rng.standard_normal(shape)
    v = oracle.newton_schulz(u)
    assert _rel(v, _spectral(u)) < 1e-10


def test_ns_transpose_equivariance_and_scale_invariance():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((12, 30))
    v = oracle.newton_schulz(u)
    assert _rel(oracle.newton_schulz(u.T), v.T) < 1e-13
    assert _rel(oracle.newton_schulz(u * 1e3), v) < 1e-6


def test_ns_orthogonal_equivariance():
    rng = np.random.default_rng(3)
    u = rng.standard_normal((10, 22))
    P, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    R, _ = np.linalg.qr(rng.standard_normal((22, 22)))
    assert _rel(oracle.newton_schulz(P @ u @ R), P @ oracle.newton_schulz(u) @ R) < 1e-11


def test_ns_special_cases():
    assert np.all(oracle.newton_schulz(np.zeros((6, 9))) == 0)
    rng = np.random.default_rng(4)
    Q, _ = np.linalg.qr(rng.standard_normal((20, 7)))          # orthonormal columns
    Qr = Q.T                                                   # 7 x 20, orthonormal rows
    v = oracle.newton_schulz(Qr)
    eps = F32(1e-7)
    s = 1.0 / (np.sqrt(7.0) + eps)
    assert _rel(v, _p5(s) * Qr) < 1e-12
    d = np.array([3.0, 1.0, 0.5, 0.1])
    v = oracle.newton_schulz(np.diag(d))
    assert _rel(v, np.diag(_p5(d / (np.linalg.norm(d) + eps)))) < 1e-12


def test_ns_output_band():
    """p^5 maps every normalised singular value >= 0.01 into [0.68, 1.14] and
    any value >= 0.002 into [0.68, 1.21]: the expected band of the output."""
    s = np.linspace(0.01, 1.0, 200001)
    y = _p5(s)
    assert y.min() > 0.68 and y.max() < 1.135
    s = np.linspace(0.002, 1.0, 200001)
    y = _p5(s)
    assert y.min() > 0.68 and y.max() < 1.2025
    rng = np.random.default_rng(5)
    u = rng.standard_normal((32, 128))
    sv = np.linalg.svd(oracle.newton_schulz(u), compute_uv=False)
    sin = np.linalg.svd(u / np.linalg.norm(u), compute_uv=False)
    assert np.all(sin > 0.01)
    assert sv.min() > 0.68 and sv.max() < 1.135


def test_muon_unit_update_rule():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((8, 24)) * 0.02).astype(np.float32)
    g = (rng.standard_normal((8, 24)) * 1e-3).astype(np.float32)
    m = np.zeros_like(w)
    hp = oracle.OracleHyper()
    w1, m1, v = oracle.muon_update_unit(w, g, m, hp)
    assert np.array_equal(m1, g)
    exp = w.astype(np.float64) - F32(0.02) * _spectral(oracle.bf16_rne(g)).astype(np.float32)
    assert np.max(np.abs(w1 - exp)) < 1e-8
    # zero gradient from a zero state leaves w bit-identical
    w2, _, v2 = oracle.muon_update_unit(w, np.zeros_like(g), m, hp)
    assert np.array_equal(w2, w) and np.all(v2 == 0)


def test_muon_scale_modes():
    assert oracle.muon_scale(0, 10, 40) == 1.0
    assert oracle.muon_scale(1, 40, 10) == 2.0
    assert oracle.muon_scale(1, 10, 40) == 1.0
    assert abs(oracle.muon_scale(2, 25, 100) - 2.0) < 1e-15


# ----------------------------------------------------------------- AdamW
ADAM = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def test_adamw_first_step_closed_form():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal(4096) * 0.02).astype(np.float32)
    g = (rng.standard_normal(4096) * 1e-3).astype(np.float32)
    z = np.zeros_like(w)
    w1, m1, v1 = oracle.adamw_step(w, g, z, z, 1, **ADAM)
    lr, wd, eps = F32(1e-3), F32(0.1), F32(1e-8)
    ref = w * (1 - lr * wd) - lr * g.astype(np.float64) / (np.abs(g.astype(np.float64)) + eps)
    assert np.max(np.abs(w1 - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_adamw_constant_gradient_closed_form():
    rng = np.random.default_rng(8)
    w0 = (rng.standard_normal(2048) * 0.02).astype(np.float32)
    g = (rng.standard_normal(2048) * 1e-3).astype(np.float32)
    w, m, v = w0, np.zeros_like(w0), np.zeros_like(w0)
    lr, wd, eps = F32(1e-3), F32(0.1), F32(1e-8)
    rho = 1 - lr * wd
    s = g.astype(np.float64) / (np.abs(g.astype(np.float64)) + eps)
    for t in range(1, 11):
        w, m, v = oracle.adamw_step(w, g, m, v, t, **ADAM)
        ref = rho ** t * w0.astype(np.float64) - lr * s * (1 - rho ** t) / (1 - rho)
        assert np.max(np.abs(w - ref)) <= 2e-6 * np.max(np.abs(ref))


def _golden_adamw():
    from fractions import Fraction
    path = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden", "adamw.txt")
    rows = []
    for ln in open(path):
        f = ln.split("#", 1)[0].split()
        if f and f[0] == "adamw":
            rows.append((int(f[1]), float(f[2]), *(Fraction(x) for x in f[3:6])))
    return rows


def test_adamw_hand_worked_three_steps():
    """Three steps worked by hand with exactly representable hyper-parameters
    (tests/golden/adamw.txt): m and v exactly, w to float32 rounding."""
    rows = _golden_adamw()
    assert [r[0] for r in rows] == [1, 2, 3]
    hp = dict(lr=0.5, beta1=0.5, beta2=0.75, eps=0.0, weight_decay=0.25)
    w, m, v = np.float32([1.0]), np.float32([0.0]), np.float32([0.0])
    for t, g, m_exp, v_exp, w_exp in rows:
        w, m, v = oracle.adamw_step(w, np.float32([g]), m, v, t, **hp)
        assert m[0] == float(m_exp) and v[0] == float(v_exp), t
        assert abs(float(w[0]) - float(w_exp)) <= 2 ** -24 * abs(float(w_exp)), t


def _adam_sums(w0, gs, t, lr, b1, b2, eps, wd):
    """AdamW after t steps in its explicit-sum form: m_t = (1-b1) sum b1^(t-k) g_k,
    v_t = (1-b2) sum b2^(t-k) g_k^2, and w_t = rho^t w0 - lr sum rho^(t-k)
    mhat_k / (sqrt(vhat_k) + eps) with rho = 1 - lr wd (every mhat_k, vhat_k
    from the sums, not from a recurrence)."""
    lr, b1, b2, eps, wd = (np.float64(np.float32(x)) for x in (lr, b1, b2, eps, wd))
    rho = 1.0 - lr * wd
    G = [np.asarray(g, np.float64) for g in gs[:t]]
    w = rho ** t * np.asarray(w0, np.float64)
    for k in range(1, t + 1):
        mk = (1 - b1) * sum(b1 ** (k - j) * G[j - 1] for j in range(1, k + 1))
        vk = (1 - b2) * sum(b2 ** (k - j) * G[j - 1] ** 2 for j in range(1, k + 1))
        w = w - lr * rho ** (t - k) * (mk / (1 - b1 ** k)) / (np.sqrt(vk / (1 - b2 ** k)) + eps)
    m = (1 - b1) * sum(b1 ** (t - j) * G[j - 1] for j in range(1, t + 1))
    v = (1 - b2) * sum(b2 ** (t - j) * G[j - 1] ** 2 for j in range(1, t + 1))
    return w, m, v


def _adam_variant(w, g, m, v, t, lr, beta1, beta2, eps, weight_decay, swap=False, no_one_minus=False,
                  abs_not_square=False, decay_after=False):
    """AdamW with one planted mistake (for checking that the pins catch it)."""
    lr, b1, b2, ep, wd = (np.float64(np.float32(x)) for x in (lr, beta1, beta2, eps, weight_decay))
    if swap:
        b1, b2 = b2, b1
    w, g, m, v = (np.asarray(x, np.float64) for x in (w, g, m, v))
    if not decay_after:
        w = w - lr * wd * w
    m = b1 * m + (1.0 if no_one_minus else 1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * (np.abs(g) if abs_not_square else g * g)
    w = w - lr * (m / (1 - b1 ** t)) / (np.sqrt(v / (1 - b2 ** t)) + ep)
    if decay_after:
        w = w - lr * wd * w
    return w, m, v


def _run_varying(step_fn, w0, gs, T):
    w, m, v = w0, np.zeros_like(w0), np.zeros_like(w0)
    out = []
    for t in range(1, T + 1):
        w, m, v = step_fn(w, gs[t - 1], m, v, t)
        out.append((np.asarray(w), np.asarray(m), np.asarray(v)))
    return out


def _varying_pin_error(out, w0, gs, hp):
    """Worst normwise distance of (w, m, v) after each step from the sum forms."""
    worst = 0.0
    for t, (w, m, v) in enumerate(out, 1):
        ws, ms, vs = _adam_sums(w0, gs, t, **hp)
        for got, ref in ((w, ws), (m, ms), (v, vs)):
            worst = max(worst, np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    return worst


def test_adamw_varying_gradient_matches_sum_forms():
    """A fresh gradient every step (magnitudes spread over two decades): the
    oracle's w, m and v after each of 8 steps equal the explicit-sum forms to
    float32 storage rounding."""
    rng = np.random.default_rng(11)
    w0 = (rng.standard_normal(2048) * 0.02).astype(np.float32)
    gs = [(rng.standard_normal(2048) * 1e-3 * 10 ** rng.uniform(-1, 1, 2048)).astype(np.float32) for _ in range(8)]
    hp = dict(lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
    out = _run_varying(lambda w, g, m, v, t: oracle.adamw_step(w, g, m, v, t, **ADAM), w0, gs, 8)
    assert _varying_pin_error(out, w0, gs, hp) <= 1e-6


def test_adamw_varying_gradient_pin_catches_planted_mistakes():
    """Mistakes a constant gradient cannot see (bias correction cancels them)
    fail the varying-gradient pin; the correct form passes it."""
    rng = np.random.default_rng(12)
    w0 = (rng.standard_normal(1024) * 0.02).astype(np.float32)
    gs = [(rng.standard_normal(1024) * 1e-3 * 10 ** rng.uniform(-1, 1, 1024)).astype(np.float32) for _ in range(6)]
    hp = dict(lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
    good = _run_varying(lambda w, g, m, v, t: _adam_variant(w, g, m, v, t, **ADAM), w0, gs, 6)
    assert _varying_pin_error(good, w0, gs, hp) <= 1e-9
    g_const = [gs[0]] * 6
    for bad in (dict(swap=True), dict(no_one_minus=True), dict(abs_not_square=True), dict(decay_after=True)):
        out = _run_varying(lambda w, g, m, v, t: _adam_variant(w, g, m, v, t, **ADAM, **bad), w0, gs, 6)
        assert _varying_pin_error(out, w0, gs, hp) > 2e-6, bad     # beyond the pin's 1e-6
    # the swap passes a constant gradient's w (m-hat = g, v-hat = g^2 whatever the betas) -- which is why
    # the varying pin exists
    out = _run_varying(lambda w, g, m, v, t: _adam_variant(w, g, m, v, t, **ADAM, swap=True), w0, g_const, 6)
    ws, _, _ = _adam_sums(w0, g_const, 6, **hp)
    assert np.max(np.abs(out[-1][0] - ws)) <= 1e-9 * np.max(np.abs(ws))


def test_adamw_zero_grad_decay_and_padding():
    w0 = np.float32([0.5, -0.25, 0.0, 0.0])
    z = np.zeros(4, np.float32)
    w = w0
    m = v = z
    for t in range(1, 6):
        w, m, v = oracle.adamw_step(w, z, m, v, t, **ADAM)
    rho = 1 - F32(1e-3) * F32(0.1)
    assert np.allclose(w, w0 * rho ** 5, rtol=1e-6, atol=0)
    assert w[2] == 0 and w[3] == 0 and not np.signbit(w[2])
    with pytest.raises(ValueError):
        oracle.adamw_step(w, z, m, v, 0, **ADAM)


# ----------------------------------------------------------------- planted mistakes
def _ns_variant(u, flip_b=False, right_product=False, no_norm=False, steps=5):
    a, b, c = F32(A), F32(B), F32(C)
    if flip_b:
        b = -b
    X = np.asarray(u, dtype=np.float64)
    if not no_norm:
        X = X / (np.linalg.norm(X) + F32(1e-7))
    for _ in range(steps):
        Am = X @ X.T
        Bm = b * Am + c * (Am @ Am)
        X = a * X + (X @ Bm if right_product else Bm @ X)
    return X


def test_pins_catch_planted_ns_mistakes():
    """The spectral pin separates the iteration from plausible mistakes."""
    rng = np.random.default_rng(9)
    u = rng.standard_normal((24, 24)) * 0.05
    ref = _spectral(u)
    assert _rel(_ns_variant(u), ref) < 1e-10           # the correct variant passes
    for bad in (dict(flip_b=True), dict(right_product=True), dict(no_norm=True)):
        assert _rel(_ns_variant(u, **bad), ref) > 1e-3, bad


def test_pins_catch_dropped_bias_correction():
    rng = np.random.default_rng(10)
    w = (rng.standard_normal(256) * 0.02).astype(np.float32)
    g = (rng.standard_normal(256) * 1e-3).astype(np.float32)
    z = np.zeros_like(w)
    lr, wd, eps = F32(1e-3), F32(0.1), F32(1e-8)
    ref = w * (1 - lr * wd) - lr * g.astype(np.float64) / (np.abs(g.astype(np.float64)) + eps)
    # the same update without bias correction differs from the closed form
    m = 0.1 * g.astype(np.float64)
    v = 0.05 * g.astype(np.float64) ** 2
    bad = w * (1 - lr * wd) - lr * m / (np.sqrt(v) + eps)
    assert np.max(np.abs(bad - ref)) > 1e-6 * np.max(np.abs(ref))
