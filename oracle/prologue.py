"""Gate and q/k preprocessing ahead of the KDA recurrence, in fp64 -- test
infrastructure only.

What is computed:
  * the lower-bounded gate of K3 (K3-on-TPU essay, blog.higcp.com, "KDA +
    Gated MLA", lower-bounded decay): per key channel
        g = g_min * sigmoid(exp(A) * z),   alpha = exp(g),   g_min = -5,
    with z the gate branch's pre-activation and A a per-head log-scale;
  * the scalar write strength beta = sigmoid(b), b the pre-activation of
    its linear branch, and L2 normalisation of q and k per token and head
    (Kimi K3 architecture walkthrough, mhpq.cn/news/56770, the Q/K
    preprocessing paragraph after "KDA 到底在算什么": q and k are
    L2-normalised, one sigmoid branch gives the per-channel forget gate,
    another the scalar beta).
The pages name no epsilon for the L2 norm; the reading used is
x / sqrt(sum(x^2) + 1e-6).  The short causal convolution and Swish that the
walkthrough puts before the normalisation are not part of this prologue.

Shapes: q, k, z [T, H, d_k]; b [T, H]; A_log [H].
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .recurrence import kda_recurrent

G_MIN = -5.0
L2_EPS = 1e-6


def sigmoid(x):
    x = np.asarray(x, np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def kda_gate(z, A_log, g_min: float = G_MIN) -> np.ndarray:
    """g = g_min * sigmoid(exp(A_log[h]) * z) for z [..., H, d_k]."""
    z = np.asarray(z, np.float64)
    scale = np.exp(np.asarray(A_log, np.float64))[:, None]
    return g_min * sigmoid(scale * z)


def l2_normalise(x) -> np.ndarray:
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2_EPS)


def kda_prologue(q, k, z, A_log, b) -> Tuple[np.ndarray, ...]:
    """(q, k, g, beta) that the recurrence consumes."""
    return l2_normalise(q), l2_normalise(k), kda_gate(z, A_log), sigmoid(b)


def kda_gated_recurrent(q, k, v, z, A_log, b, S0=None):
    """The prologue, then the token recurrence: o [T, H, d_v], S_T."""
    qn, kn, g, beta = kda_prologue(q, k, z, A_log, b)
    return kda_recurrent(qn, kn, v, g, beta, S0)
