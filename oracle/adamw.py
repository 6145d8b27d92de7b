"""AdamW for 1-D and elementwise units (oracle; test infrastructure only).

[SS-HSDP §5.2]: Muon updates most parameters and AdamW updates the remainder;
[SS-HSDP Appendix B.1]: AdamW is the optimiser of all performance runs.  The
pages do not write AdamW out.  Reading taken: decoupled weight decay scaled by
the learning rate and applied to the pre-update weight, bias-corrected moments,
epsilon added after the square root:

    w <- w - lr*wd*w
    m <- b1*m + (1-b1)*g
    v <- b2*v + (1-b2)*g*g
    w <- w - lr * (m / (1-b1**t)) / (sqrt(v / (1-b2**t)) + eps)

with step t >= 1 supplied by the caller.  float64 arithmetic on the float32
inputs; results stored to float32 with round-to-nearest-even.
"""

import numpy as np


def adamw_step(w, g, m, v, t, lr, beta1, beta2, eps, weight_decay):
    if t < 1:
        raise ValueError("AdamW step counter must be >= 1")
    lr, b1, b2, ep, wd = (np.float64(np.float32(x)) for x in (lr, beta1, beta2, eps, weight_decay))
    w = w.astype(np.float64)
    g = g.astype(np.float64)
    m = m.astype(np.float64)
    v = v.astype(np.float64)
    w = w - lr * wd * w
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * g * g
    mhat = m / (1.0 - b1 ** t)
    vhat = v / (1.0 - b2 ** t)
    w = w - lr * mhat / (np.sqrt(vhat) + ep)
    return w.astype(np.float32), m.astype(np.float32), v.astype(np.float32)
