"""Brute-force KDA via explicit transition matrices -- test infrastructure.

Takes the update exactly as the equation prints it (Kimi K3 architecture
walkthrough, mhpq.cn/news/56770, "KDA 到底在算什么"):

    A_t = (I - beta_t k_t k_t^T) Diag(alpha_t)        a full d_k x d_k matrix
    S_t = A_t S_{t-1} + beta_t k_t v_t^T

and evaluates its closed form without any running state:

    S_t = (A_t ... A_1) S0 + sum_{s<=t} (A_t ... A_{s+1}) beta_s k_s v_s^T
    o_t = S_t^T q_t

Every product is rebuilt from scratch for every t (O(T^2) matrix products),
so a mistake in the rank-1 bookkeeping of the recurrence cannot hide here.
Tiny inputs only.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def _transitions(k, g, beta):
    T, dk = k.shape
    I = np.eye(dk)
    return [(I - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t]))
            for t in range(T)]


def _chain_product(A, lo, hi, dk):
    """A_{hi-1} ... A_{lo} (identity when lo >= hi); indices are 0-based."""
    P = np.eye(dk)
    for s in range(lo, hi):
        P = A[s] @ P
    return P


def kda_transition_bruteforce(q, k, v, g, beta, S0: Optional[np.ndarray] = None
                              ) -> Tuple[np.ndarray, np.ndarray]:
    """Single head. q, k, g : [T, dk]; v : [T, dv]; beta : [T];
    S0 : [dk, dv] or None.  Returns o [T, dv] and S_T [dk, dv] (fp64)."""
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64)
    A = _transitions(k, g, beta)
    o = np.zeros((T, dv))
    S_t = S0
    for t in range(T):
        S_t = _chain_product(A, 0, t + 1, dk) @ S0
        for s in range(t + 1):
            S_t = S_t + _chain_product(A, s + 1, t + 1, dk) @ (beta[s] * np.outer(k[s], v[s]))
        o[t] = S_t.T @ q[t]
    return o, S_t
