"""Reverse-mode gradients of the KDA token recurrence in fp64 -- test
infrastructure only.

The forward map is the recurrence of the Kimi K3 architecture walkthrough
(mhpq.cn/news/56770, "KDA 到底在算什么"), in the rank-1 form of
recurrence.py:  S'_t = Diag(exp(g_t)) S_{t-1};  w_t = S'_t^T k_t;
u_t = beta_t (v_t - w_t);  S_t = S'_t + k_t u_t^T;  o_t = S_t^T q_t.
Given cotangents dO of o and dS_T of the final state, the function below
walks the tokens backwards applying the chain rule to each of those five
lines in turn, with dS the cotangent of S_t:

    dS    += q_t dO_t^T              dq_t  = S_t dO_t
    du     = dS^T k_t                dk_t  = dS u_t
    dv_t   = beta_t du               dbeta_t = (v_t - w_t) . du
    dw     = -beta_t du              dS'   = dS + k_t dw^T,  dk_t += S'_t dw
    dg_t   = rowsum(dS' * S'_t)      dS    = Diag(exp(g_t)) dS'

and returns dS_0 at the end.  A backward pass (custom VJP) is part of the
KDA kernel suite the K3-on-TPU essay describes (blog.higcp.com, the section
on the existing TPU kernel).  Plain loops over tokens; all states kept.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def kda_recurrent_vjp(q, k, v, g, beta, dO, S0: Optional[np.ndarray] = None,
                      dST: Optional[np.ndarray] = None) -> Tuple[np.ndarray, ...]:
    """One sequence, all heads.  q, k, g [T, H, dk]; v, dO [T, H, dv];
    beta [T, H]; S0, dST [H, dk, dv] or None.
    Returns dq, dk, dv, dg, dbeta, dS0 (fp64, the inputs' shapes)."""
    q, k, v, g, beta, dO = (np.asarray(x, np.float64) for x in (q, k, v, g, beta, dO))
    T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv)) if S0 is None else np.array(S0, np.float64, copy=True)
    Sp = np.zeros((T, H, dk, dv))        # S'_t
    Sn = np.zeros((T, H, dk, dv))        # S_t
    W = np.zeros((T, H, dv))
    U = np.zeros((T, H, dv))
    for t in range(T):
        Sp[t] = S * np.exp(g[t])[:, :, None]
        W[t] = np.einsum("hij,hi->hj", Sp[t], k[t])
        U[t] = beta[t][:, None] * (v[t] - W[t])
        S = Sp[t] + k[t][:, :, None] * U[t][:, None, :]
        Sn[t] = S
    dq, dkk, dvv, dg = (np.zeros_like(x) for x in (q, k, v, g))
    db = np.zeros_like(beta)
    dS = np.zeros((H, dk, dv)) if dST is None else np.array(dST, np.float64, copy=True)
    for t in range(T - 1, -1, -1):
        dS = dS + q[t][:, :, None] * dO[t][:, None, :]
        dq[t] = np.einsum("hij,hj->hi", Sn[t], dO[t])
        du = np.einsum("hij,hi->hj", dS, k[t])
        dkk[t] = np.einsum("hij,hj->hi", dS, U[t])
        dvv[t] = beta[t][:, None] * du
        db[t] = np.sum((v[t] - W[t]) * du, axis=-1)
        dw = -beta[t][:, None] * du
        dSp = dS + k[t][:, :, None] * dw[:, None, :]
        dkk[t] += np.einsum("hij,hj->hi", Sp[t], dw)
        dg[t] = np.sum(dSp * Sp[t], axis=-1)
        dS = dSp * np.exp(g[t])[:, :, None]
    return dq, dkk, dvv, dg, db, dS


def kda_recurrent_vjp_varlen(q, k, v, g, beta, dO, cu_seqlens, S0=None, dST=None):
    """Packed batch: every sequence is independent (its own S0 and dS_T)."""
    cu = np.asarray(cu_seqlens, np.int64)
    n = len(cu) - 1
    outs = [np.zeros(np.shape(x)) for x in (q, k, v, g, beta)]
    H, dk = np.shape(q)[1:]
    dv = np.shape(v)[-1]
    dS0 = np.zeros((n, H, dk, dv))
    for s in range(n):
        a, b = cu[s], cu[s + 1]
        r = kda_recurrent_vjp(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], dO[a:b],
                              None if S0 is None else S0[s], None if dST is None else dST[s])
        for o_, x in zip(outs, r[:5]):
            o_[a:b] = x
        dS0[s] = r[5]
    return (*outs, dS0)
