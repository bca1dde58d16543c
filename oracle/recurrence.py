"""fp64 token-by-token KDA recurrence (NumPy) -- test infrastructure only.

Definition (Kimi K3 architecture walkthrough, mhpq.cn/news/56770, section
"KDA 到底在算什么", state-update equation; step order from the figure
caption there: per-channel decay, then erase along the current key, then
write; the read uses the updated state):

    S' = Diag(exp(g_t)) S_{t-1}              rows = key channels
    u  = beta_t (v_t - S'^T k_t)             delta against the decayed state
    S_t = S' + k_t u^T                        = (I - b k k^T) S' + b k v^T
    o_t = S_t^T q_t

No attention scale is applied to q (the equation has none).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def kda_recurrent(q, k, v, g, beta, S0: Optional[np.ndarray] = None
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """One sequence, all heads at once.

    q, k, g : [T, H, dk]    v : [T, H, dv]    beta : [T, H]
    S0      : [H, dk, dv] or None (zeros)
    returns o [T, H, dv] fp64 and S_T [H, dk, dv] fp64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv)) if S0 is None else np.array(S0, np.float64, copy=True)
    o = np.zeros((T, H, dv))
    for t in range(T):
        S *= np.exp(g[t])[:, :, None]                         # decay rows
        w = np.einsum("hij,hi->hj", S, k[t])                  # S'^T k
        u = beta[t][:, None] * (v[t] - w)                     # delta
        S += k[t][:, :, None] * u[:, None, :]                 # rank-1 write
        o[t] = np.einsum("hij,hi->hj", S, q[t])               # read
    return o, S


def kda_recurrent_varlen(q, k, v, g, beta, cu_seqlens, S0=None
                         ) -> Tuple[np.ndarray, np.ndarray]:
    """Packed batch: sequences are cu_seqlens[n]:cu_seqlens[n+1]; each one
    starts from its own S0[n] (or zeros) and never sees the others.
    Returns o [N, H, dv] and S_T [n_seqs, H, dk, dv]."""
    cu = np.asarray(cu_seqlens, np.int64)
    n_seqs = len(cu) - 1
    N, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    o = np.zeros((N, H, dv))
    ST = np.zeros((n_seqs, H, dk, dv))
    for n in range(n_seqs):
        a, b = cu[n], cu[n + 1]
        s0 = None if S0 is None else S0[n]
        o[a:b], ST[n] = kda_recurrent(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], s0)
    return o, ST


def kda_decode_step(q, k, v, g, beta, S) -> Tuple[np.ndarray, np.ndarray]:
    """A single token for a batch of independent chains: the recurrence with
    T = 1.  q, k, g : [N, H, dk]; v : [N, H, dv]; beta : [N, H];
    S : [N, H, dk, dv].  Returns (o [N, H, dv], S_new) without touching S."""
    q = np.asarray(q, np.float64)
    N, H, dk = q.shape
    dv = np.shape(v)[-1]
    o, ST = kda_recurrent(q.reshape(1, N * H, dk),
                          np.asarray(k, np.float64).reshape(1, N * H, dk),
                          np.asarray(v, np.float64).reshape(1, N * H, dv),
                          np.asarray(g, np.float64).reshape(1, N * H, dk),
                          np.asarray(beta, np.float64).reshape(1, N * H),
                          np.asarray(S, np.float64).reshape(N * H, dk, dv))
    return o.reshape(N, H, dv), ST.reshape(N, H, dk, dv)
