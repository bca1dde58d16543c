"""fp64 chunked (WY/UT) form of KDA -- test infrastructure only.

The pages only sketch the chunked form: keys are rescaled by the reciprocal
of the cumulative decay, and the lower bound g >= -5 keeps the cumulative
log-decay of a 16-token tile inside (-80, 0) so that both the diagonal and
off-diagonal tiles can be dense matrix products (K3-on-TPU essay,
blog.higcp.com, section "KDA + Gated MLA", lower-bounded decay; Kimi K3
architecture walkthrough, mhpq.cn/news/56770, the lower-bounded-decay
section).  The algebra below is derived from the token recurrence; this
module checks it in fp64 before any kernel relies on it.  Parity of the HIP
path is always measured against the token recurrence, not against this.

For one chunk of n tokens with entry state S, per key channel c let
Gc_r = g_1 + ... + g_r (inclusive, relative to the chunk start).  Then

    u_r = beta_r (v_r - S^T (k_r e^{Gc_r})
                  - sum_{i<r} [ (k_r e^{Gc_r}) . (k_i e^{-Gc_i}) ] u_i)

which in matrix form is (I + A) U = Diag(beta) (V - Kt S) with
A_ri = beta_r Kt_r . Kh_i  (i < r),  Kt = k e^{Gc},  Kh = k e^{-Gc}.  Hence

    T  = (I + A)^{-1} Diag(beta)        (unit lower-triangular solve)
    U  = T (V - Kt S)
    O  = Qt S + P U,   P_ri = Qt_r . Kh_i (i <= r),   Qt = q e^{Gc}
    S' = Diag(e^{Gc_n}) S + Kd^T U,     Kd = k e^{Gc_n - Gc}

Inside the products Kt_r . Kh_i every 16-token row tile a uses its own
reference ref_a (the cumulative log-decay just before the tile), i.e. it
multiplies (k_r e^{Gc_r - ref_a}) by (k_i e^{ref_a - Gc_i}); each exponent
then stays in [-80, 0] or [0, 80] when g >= -5.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np
from scipy.linalg import solve_triangular

TILE = 16


def _chunk(q, k, v, g, beta, S):
    n = k.shape[0]
    Gc = np.cumsum(g, axis=0)                       # [n, dk], inclusive
    A = np.zeros((n, n))
    P = np.zeros((n, n))
    for a0 in range(0, n, TILE):
        rows = slice(a0, min(a0 + TILE, n))
        ref = Gc[a0 - 1] if a0 > 0 else np.zeros(Gc.shape[1])
        Lk = k[rows] * np.exp(Gc[rows] - ref)       # exponent in [-80, 0]
        Lq = q[rows] * np.exp(Gc[rows] - ref)
        cols = slice(0, rows.stop)
        R = k[cols] * np.exp(ref - Gc[cols])        # <= 80 inside the tile
        A[rows, cols] = Lk @ R.T
        P[rows, cols] = Lq @ R.T
    A = np.tril(A, -1) * beta[:, None]
    P = np.tril(P, 0)
    Kt = k * np.exp(Gc)
    Qt = q * np.exp(Gc)
    Kd = k * np.exp(Gc[-1] - Gc)
    T = solve_triangular(np.eye(n) + A, np.diag(beta), lower=True,
                         unit_diagonal=True)
    U = T @ (v - Kt @ S)
    O = Qt @ S + P @ U
    S_new = np.exp(Gc[-1])[:, None] * S + Kd.T @ U
    return O, S_new


def kda_chunked(q, k, v, g, beta, S0: Optional[np.ndarray] = None,
                chunk: int = 16) -> Tuple[np.ndarray, np.ndarray]:
    """Single head. q, k, g : [T, dk]; v : [T, dv]; beta : [T]; S0 : [dk, dv]
    or None.  ``chunk`` must be a multiple of 16.  Returns o [T, dv] and
    S_T [dk, dv] in fp64."""
    if chunk % TILE:
        raise ValueError("chunk must be a multiple of 16")
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64, copy=True)
    o = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        c1 = min(c0 + chunk, T)
        o[c0:c1], S = _chunk(q[c0:c1], k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1], S)
    return o, S
