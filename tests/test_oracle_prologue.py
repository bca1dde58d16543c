"""CPU pins of the prologue oracle (oracle/prologue.py) against facts from
outside it: exact sigmoid values, the gate's bound, the log-scale's
meaning, scale invariance of L2 normalisation, and the composition with the
independent C recurrence."""
import math

import numpy as np

from oracle import clib
from oracle.prologue import (L2_EPS, kda_gate, kda_gated_recurrent, kda_prologue,
                             l2_normalise)


def test_gate_exact_values():
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    z = np.array([[[0.0, math.log(3.0), -math.log(3.0)]]])
    g = kda_gate(z, np.array([0.0]))
    assert np.allclose(g, [[[-2.5, -3.75, -1.25]]], rtol=0, atol=1e-15)


def test_gate_bounds_and_monotone():
    z = np.linspace(-40, 40, 2001)[None, None, :]
    g = kda_gate(z, np.array([0.3]))
    assert np.all(g >= -5.0) and np.all(g <= 0.0)
    assert np.all(np.diff(g[0, 0]) <= 0)          # larger z: stronger decay
    assert g[0, 0, 0] > -1e-12 and g[0, 0, -1] < -5.0 + 1e-12


def test_gate_log_scale_doubles_z():
    """exp(A + ln 2) z = exp(A) (2 z): the per-head scale is a log-scale."""
    r = np.random.default_rng(0)
    z = r.standard_normal((7, 3, 16))
    A = r.standard_normal(3)
    assert np.allclose(kda_gate(z, A + math.log(2.0)), kda_gate(2.0 * z, A), rtol=0, atol=1e-14)


def test_l2_unit_norm_and_scale_invariance():
    r = np.random.default_rng(1)
    x = r.standard_normal((5, 2, 32)) * 10
    n = np.linalg.norm(l2_normalise(x), axis=-1)
    assert np.allclose(n, 1.0, atol=1e-8)
    assert np.allclose(l2_normalise(3.7 * x), l2_normalise(x), atol=1e-8)
    # the epsilon keeps a zero vector finite
    assert np.all(l2_normalise(np.zeros((1, 1, 8))) == 0.0)
    assert L2_EPS == 1e-6


def test_gated_recurrence_matches_c_oracle_on_prologue_outputs():
    r = np.random.default_rng(2)
    T, H, dk, dv = 40, 2, 16, 8
    q, k, z = (r.standard_normal((T, H, dk)) for _ in range(3))
    v = r.standard_normal((T, H, dv))
    b = r.standard_normal((T, H))
    A = r.standard_normal(H) * 0.5
    o, S = kda_gated_recurrent(q, k, v, z, A, b)
    qn, kn, g, beta = kda_prologue(q, k, z, A, b)
    f = lambda x: np.asarray(x, np.float32)               # noqa: E731
    o_c, S_c, _ = clib.fwd(f(qn), f(kn), f(v), f(g), f(beta), np.array([0, T], np.int32))
    # the C oracle reads fp32 inputs: agreement to fp32 input rounding
    assert np.max(np.abs(o - o_c)) < 1e-5 and np.max(np.abs(S - S_c)) < 1e-5
