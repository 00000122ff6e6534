"""Reference linear layer (oracle).

y = x . w_hat^T with x [M][K] and the dequantized weights w_hat [N][K], both
holding 16-bit values (exact in fp64), evaluated in fp64.  This is the
product that W4A16 performs after dequantizing the weights back to 16 bits
([P1] section 5 opening; [P2] section 十一; [P4] section 1.2: decode is bound
by moving the weights).

Acceptance for float outputs: max|y - y_ref| / max|y_ref| over one output
tensor, compared against a tolerance stated by the caller.
"""

import numpy as np


def reference(x, w_hat):
    """fp64 y = x . w_hat^T (NumPy matmul, a textbook BLAS routine)."""
    return np.asarray(x, np.float64) @ np.asarray(w_hat, np.float64).T


def naive(x, w_hat):
    """Triple loop, for tiny shapes only (used to pin :func:`reference`)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w_hat, np.float64)
    m, k = x.shape
    n = w.shape[0]
    y = np.zeros((m, n), dtype=np.float64)
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for t in range(k):
                acc += x[i, t] * w[j, t]
            y[i, j] = acc
    return y


def silu_gated(g, u):
    """silu(g) * u in fp64, silu(v) = v / (1 + exp(-v)): the activation
    product that joins the gate and up projections of a gated MLP block.
    The pages list the gate, up and down projections of each block ([P3]
    step 4) but name no activation; SiLU, the activation of the
    LLaMA/Qwen2-style blocks those projections belong to, is the reading
    taken here."""
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def max_rel_err(y, y_ref):
    """max|y - y_ref| / max|y_ref| (the float acceptance measure)."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    den = np.abs(y_ref).max()
    if den == 0:
        return float(np.abs(y).max())
    return float(np.abs(y - y_ref).max() / den)
