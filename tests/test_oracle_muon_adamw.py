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
