"""Pins for the KDA oracle: facts fixed by the pages or by mathematics, each
written as a predicate over an implementation

    impl(q [T,dk], k [T,dk], v [T,dv], g [T,dk], beta [T], S0 [dk,dv] | None)
        -> (o [T,dv], S_T [dk,dv])

so that the same predicates can be run on every oracle formulation and on
deliberately broken copies of the recurrence (tests/test_oracle_mutants.py),
which must each fail at least one of them.

The equation pinned is the KDA state update of the Kimi K3 architecture
walkthrough (mhpq.cn/news/56770), section "KDA 到底在算什么", with
alpha = exp(g) per key channel (K3-on-TPU essay, blog.higcp.com, "KDA +
Gated MLA", lower-bounded decay).
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-10
# Every input a pin builds goes through QUANT before it is used, both by the
# implementation and by the closed form, so that an implementation that reads
# fp32 inputs can be pinned on exactly the values it sees (see fp32_inputs).
QUANT = lambda x: np.asarray(x, np.float64)


class fp32_inputs:
    """Context manager: round pin inputs to fp32 and loosen TOL to 2e-6."""

    def __enter__(self):
        global QUANT, TOL
        self._old = (QUANT, TOL)
        QUANT = lambda x: np.asarray(np.asarray(x, np.float32), np.float64)
        TOL = 2e-6
        return self

    def __exit__(self, *exc):
        global QUANT, TOL
        QUANT, TOL = self._old
        return False


def _qz(*xs):
    return tuple(None if x is None else QUANT(x) for x in xs)


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_case(seed, T=24, dk=6, dv=4, s0=True, gmin=-5.0):
    r = _rng(seed)
    q = _unit(r.standard_normal((T, dk)))
    k = _unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    g = r.uniform(gmin, 0.0, (T, dk))
    beta = r.uniform(0.0, 1.0, T)
    S0 = r.standard_normal((dk, dv)) if s0 else None
    return _qz(q, k, v, g, beta, S0)


def close(a, b, tol=None):
    tol = TOL if tol is None else max(tol, TOL)
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return a.shape == b.shape and np.all(np.isfinite(a)) and \
        float(np.max(np.abs(a - b), initial=0.0)) <= tol * max(1.0, float(np.max(np.abs(b), initial=0.0)))


# ---------------------------------------------------------------------------
def pin_hand_example(impl):
    """Hand-derived two-token example (tests/golden/hand_example.json)."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        ex = json.load(f)
    q, k, v, g, beta = _qz(ex["q"], ex["k"], ex["v"], np.log(np.asarray(ex["alpha"])),
                           ex["beta"])
    o, S = impl(q, k, v, g, beta, None)
    o1, S1 = impl(q[:1], k[:1], v[:1], g[:1], beta[:1], None)
    return (close(o, ex["expected_o"]) and close(S, ex["expected_S_T"])
            and close(S1, ex["expected_S1"]))


def pin_pure_decay(impl):
    """beta = 0: the erase and the write vanish and every key channel (row
    of S) keeps only its own retention: S_T = Diag(exp(sum_t g_t)) S0 and
    o_t = S0^T (exp(Gc_t) * q_t), Gc_t the inclusive cumulative log-decay."""
    ok = True
    for seed, (dk, dv) in enumerate([(6, 4), (5, 5), (3, 7)]):
        q, k, v, g, beta, S0 = random_case(100 + seed, T=20, dk=dk, dv=dv)
        beta = np.zeros_like(beta)
        o, S = impl(q, k, v, g, beta, S0)
        Gc = np.cumsum(g, axis=0)
        ok &= close(S, np.exp(Gc[-1])[:, None] * S0)
        ok &= close(o, (np.exp(Gc) * q) @ S0)
    return bool(ok)


def pin_retrieval(impl):
    """beta_t = 1 and |k_t| = 1: I - k k^T projects out k_t, so right after
    the update S_t^T k_t = v_t whatever the decay or the history.  Reading
    with q_t = k_t must therefore return v_t exactly."""
    ok = True
    for seed, (dk, dv) in enumerate([(6, 4), (4, 4), (3, 8)]):
        q, k, v, g, beta, S0 = random_case(200 + seed, T=30, dk=dk, dv=dv)
        o, _ = impl(k.copy(), k, v, g, QUANT(np.ones_like(beta)), S0)
        ok &= close(o, v)
    return bool(ok)


def pin_linear_attention(impl):
    """alpha = 1, beta = 1 and orthonormal keys (T <= d_k): no write ever
    overlaps an earlier one, so KDA reduces to causal linear attention,
    o = tril(Q K^T) V (a plain masked matrix product)."""
    ok = True
    for seed, (T, dk, dv) in enumerate([(6, 6, 4), (4, 7, 5), (8, 8, 8)]):
        r = _rng(300 + seed)
        Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
        k, q, v = _qz(Qm[:, :T].T.copy(), r.standard_normal((T, dk)),
                      r.standard_normal((T, dv)))
        o, S = impl(q, k, v, np.zeros((T, dk)), np.ones(T), None)
        ok &= close(o, np.tril(q @ k.T) @ v)
        ok &= close(S, k.T @ v)
    return bool(ok)


def pin_onehot_overwrite(impl):
    """One-hot keys k_t = e_{c_t} with beta = 1: the erase clears exactly
    row c_t of the decayed state and the write puts v_t there, so every row
    of S_T is either its last written value or S0's row, times the product
    of that channel's retentions since then (per-channel decay acts on rows)."""
    ok = True
    for seed, (T, dk, dv) in enumerate([(15, 5, 3), (12, 4, 4)]):
        r = _rng(400 + seed)
        c = r.integers(0, dk - 1, T)            # channel dk-1 is never written
        k = np.eye(dk)[c]
        q, v, g, S0 = _qz(r.standard_normal((T, dk)), r.standard_normal((T, dv)),
                          r.uniform(-3.0, 0.0, (T, dk)), r.standard_normal((dk, dv)))
        o, S = impl(q, k, v, g, np.ones(T), S0)
        want = np.empty((dk, dv))
        for ch in range(dk):
            hits = np.nonzero(c == ch)[0]
            if len(hits):
                t = hits[-1]
                want[ch] = v[t] * np.exp(g[t + 1:, ch].sum())
            else:
                want[ch] = S0[ch] * np.exp(g[:, ch].sum())
        ok &= close(S, want)
        ok &= close(o[-1], S.T @ q[-1])
    return bool(ok)


def pin_householder(impl):
    """beta = 2, alpha = 1, v = 0, unit keys: each step multiplies the state
    on the left by the Householder reflector I - 2 k k^T, so S_T is the
    product of reflectors applied to S0 and its Frobenius norm is kept."""
    ok = True
    for seed, (dk, dv) in enumerate([(5, 3), (4, 4)]):
        q, k, v, g, beta, S0 = random_case(500 + seed, T=9, dk=dk, dv=dv)
        o, S = impl(q, k, np.zeros_like(v), np.zeros_like(g), np.full_like(beta, 2.0), S0)
        H = np.eye(dk)
        for t in range(len(k)):
            H = (np.eye(dk) - 2.0 * np.outer(k[t], k[t])) @ H
        ok &= close(S, H @ S0)
        ok &= abs(np.linalg.norm(S) - np.linalg.norm(S0)) <= TOL * np.linalg.norm(S0)
    return bool(ok)


def pin_bruteforce(impl):
    """Agreement with the explicit product of d_k x d_k transition matrices
    (oracle.transition) on tiny random inputs, with a nonzero S0."""
    from oracle.transition import kda_transition_bruteforce
    ok = True
    for seed, (T, dk, dv) in enumerate([(12, 5, 3), (7, 4, 4), (16, 3, 6)]):
        case = random_case(600 + seed, T=T, dk=dk, dv=dv)
        o, S = impl(*case)
        ob, Sb = kda_transition_bruteforce(*case)
        ok &= close(o, ob, 1e-9) and close(S, Sb, 1e-9)
    return bool(ok)


def pin_contraction(impl):
    """Unit keys, beta in [0, 1], alpha <= 1 and v = 0: each transition has
    spectral norm <= 1, so |S_T|_2 <= |S0|_2."""
    ok = True
    for seed in range(3):
        q, k, v, g, beta, S0 = random_case(700 + seed, T=40, dk=6, dv=5, gmin=-0.2)
        _, S = impl(q, k, np.zeros_like(v), g, beta, S0)
        ok &= np.linalg.norm(S, 2) <= np.linalg.norm(S0, 2) * (1 + 1e-12)
    return bool(ok)


def pin_carry_over(impl):
    """Running a sequence in two segments, the second starting from the
    first one's final state, equals one run over the whole sequence."""
    ok = True
    for seed, T1 in enumerate([1, 7, 16, 23]):
        q, k, v, g, beta, S0 = random_case(800 + seed, T=40, dk=5, dv=4)
        o, S = impl(q, k, v, g, beta, S0)
        oa, Sa = impl(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], S0)
        ob, Sb = impl(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], Sa)
        ok &= close(np.concatenate([oa, ob]), o) and close(Sb, S)
    return bool(ok)


def pin_structure(impl):
    """Column independence (o[:, j] and S[:, j] depend only on v[:, j] and
    S0[:, j]), joint linearity in (S0, v), and equivariance under a
    permutation of the key channels."""
    q, k, v, g, beta, S0 = random_case(900, T=25, dk=6, dv=5)
    o, S = impl(q, k, v, g, beta, S0)
    ok = True
    v2, S02 = v.copy(), S0.copy()
    v2[:, 2] += 1.0
    S02[:, 2] -= 0.5
    o2, S2 = impl(q, k, v2, g, beta, S02)
    keep = [0, 1, 3, 4]
    ok &= close(o2[:, keep], o[:, keep]) and close(S2[:, keep], S[:, keep])
    ok &= not close(o2[:, 2], o[:, 2])
    r = _rng(901)
    vb, S0b = _qz(r.standard_normal(v.shape), r.standard_normal(S0.shape))
    ob, Sb = impl(q, k, vb, g, beta, S0b)
    oc, Sc = impl(q, k, 2.0 * v - 3.0 * vb, g, beta, 2.0 * S0 - 3.0 * S0b)
    ok &= close(oc, 2.0 * o - 3.0 * ob, 1e-9) and close(Sc, 2.0 * S - 3.0 * Sb, 1e-9)
    p = r.permutation(6)
    op, Sp = impl(q[:, p], k[:, p], v, g[:, p], beta, S0[p])
    ok &= close(op, o) and close(Sp, S[p])
    return bool(ok)


ALL_PINS = [pin_hand_example, pin_pure_decay, pin_retrieval, pin_linear_attention,
            pin_onehot_overwrite, pin_householder, pin_bruteforce, pin_contraction,
            pin_carry_over, pin_structure]
