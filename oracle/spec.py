"""Speculative-decoding verify and replay in fp64 -- test infrastructure only.

What is computed (K3-on-TPU essay, blog.higcp.com, section "KDA + Gated
MLA", the costs section, item (1)): at decode the KDA state advances in
place, so drafted tokens are first scored without committing the state, and
the accepted ones are later replayed from their cached inputs to rebuild
it.  Every step below is the token recurrence of the Kimi K3 architecture
walkthrough (mhpq.cn/news/56770, "KDA 到底在算什么"), applied by
``recurrence.kda_recurrent``; nothing here adds arithmetic of its own.

Token tensors hold K tokens per sequence: q, k, g [N, K, H, d_k];
v [N, K, H, d_v]; beta [N, K, H]; the state S is [N, H, d_k, d_v].
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .recurrence import kda_recurrent


def kda_spec_verify(q, k, v, g, beta, S) -> np.ndarray:
    """Outputs o [N, K, H, d_v] of running each sequence's K drafts from its
    state S[n] one token at a time; S itself is left as it was."""
    q = np.asarray(q, np.float64)
    N, K, H, _ = q.shape
    dv = np.shape(v)[-1]
    o = np.zeros((N, K, H, dv))
    for n in range(N):
        o[n], _ = kda_recurrent(q[n], k[n], v[n], g[n], beta[n], np.asarray(S[n], np.float64))
    return o


def kda_spec_commit(k, v, g, beta, n_accept, S) -> np.ndarray:
    """The state after replaying the first n_accept[n] (clamped into [0, K])
    cached tokens of each sequence from S[n]; returns the new [N, H, d_k,
    d_v] state (S is not modified)."""
    k = np.asarray(k, np.float64)
    N, K, H, dk = k.shape
    out = np.array(S, np.float64, copy=True)
    for n in range(N):
        a = int(min(max(int(n_accept[n]), 0), K))
        if a == 0:
            continue
        q0 = np.zeros((a, H, dk))
        _, out[n] = kda_recurrent(q0, k[n, :a], v[n, :a], g[n, :a], beta[n, :a], out[n])
    return out


def kda_spec_step(prev, n_accept, drafts, S) -> Tuple[np.ndarray, np.ndarray]:
    """One decode-loop step: commit the previous drafts' accepted prefix,
    then verify the new drafts from the committed state.  prev and drafts
    are dicts of k, v, g, beta (drafts also q).  Returns (o, new S)."""
    S1 = S if prev is None else kda_spec_commit(prev["k"], prev["v"], prev["g"], prev["beta"],
                                                n_accept, S)
    o = kda_spec_verify(drafts["q"], drafts["k"], drafts["v"], drafts["g"], drafts["beta"], S1)
    return o, S1
