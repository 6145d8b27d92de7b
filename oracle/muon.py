"""Muon update of one matrix unit: f0 momentum, f1 Newton-Schulz, f2 weight update.

[SS-HSDP §3.1, EG1]: per update unit, F = [f0, f1, f2]; f0 updates the
momentum m from the gradient g and writes a BF16 intermediate u; f1 applies
Newton-Schulz to u and writes the FP32 update direction v; f2 updates the main
weight from v.  [SS-HSDP §3.4]: only f1 needs the whole unit; f0 and f2 are
elementwise.  [SS-HSDP §1]: with per-head Muon each attention head is updated
independently.  The Newton-Schulz coefficients (a, b, c) = (3.4445, -4.7750,
2.0315), five steps on the Frobenius-normalised input, momentum 0.95 and lr 0.02
are the tiny attention block's stated settings.

Readings taken (the pages do not write the Muon formulas out; these are the
plainest forms consistent with EG1):
* momentum (heavy ball): m <- mu*m + g; u <- bf16(m).  Option nesterov:
  u <- bf16(g + mu*m_new).
* normalisation: X0 = u / (||u||_F + eps), eps = 1e-7, norm over the bf16 u;
* each step: A = X X^T; B = b A + c A A; X <- a X + B X, on the orientation with
  the smaller Gram (r = min(rows, cols)); a tall unit uses A = X^T X and
  X <- a X + X B, which is the same map (X (X^T X) = (X X^T) X);
* v = fp32(X); w <- w - lr*wd*w - lr*scale*v with wd = 0 and scale = 1 unless
  chosen otherwise (scale mode 1: sqrt(max(1, rows/cols)); mode 2:
  0.2*sqrt(max(rows, cols))).
NS runs entirely in float64 through numpy.matmul.
"""

import numpy as np

from .numerics import bf16_rne


def momentum_step(m, g, mu, nesterov=False):
    """f0: returns (m_new float32, u float32 holding bf16 values)."""
    mu = np.float64(np.float32(mu))
    m_new = (mu * m.astype(np.float64) + g.astype(np.float64)).astype(np.float32)
    src = m_new
    if nesterov:
        src = (g.astype(np.float64) + mu * m_new.astype(np.float64)).astype(np.float32)
    return m_new, bf16_rne(src)


def newton_schulz(u, steps=5, a=3.4445, b=-4.7750, c=2.0315, eps=1e-7, progress=None):
    """f1: quintic Newton-Schulz orthogonalisation of u (any 2-D shape), float64.

    The coefficients arrive as the float32 values the library receives.
    ``progress`` (optional) is called with the step number after each step
    (long runs on large units report as they go).
    """
    a, b, c = (np.float64(np.float32(t)) for t in (a, b, c))
    eps = np.float64(np.float32(eps))
    X = np.asarray(u, dtype=np.float64)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = X / (np.sqrt(np.sum(X * X)) + eps)
    for k in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
        if progress is not None:
            progress(k + 1)
    return X.T if tall else X


def muon_scale(mode, rows, cols):
    if mode == 0:
        return 1.0
    if mode == 1:
        return float(np.sqrt(max(1.0, rows / cols)))
    if mode == 2:
        return 0.2 * float(np.sqrt(max(rows, cols)))
    raise ValueError(mode)


def muon_update_unit(w, g, m, hp):
    """All of F for one unit.  ``hp`` has lr, momentum, weight_decay, nesterov,
    ns_steps, a, b, c, ns_eps, scale_mode.  Returns (w_new, m_new, v) with w_new
    and m_new float32 and v the float64 direction."""
    m_new, u = momentum_step(m, g, hp.momentum, hp.nesterov)
    v = newton_schulz(u, hp.ns_steps, hp.a, hp.b, hp.c, hp.ns_eps)
    lr = np.float64(np.float32(hp.lr))
    wd = np.float64(np.float32(hp.weight_decay))
    s = muon_scale(hp.scale_mode, *w.shape)
    v32 = v.astype(np.float32).astype(np.float64)
    w64 = w.astype(np.float64)
    w_new = (w64 - lr * wd * w64 - lr * s * v32).astype(np.float32)
    return w_new, m_new, v
