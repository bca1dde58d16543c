"""CPU pins of the backward oracle (oracle/backward.py): central finite
differences of the pinned forward oracle, the closed form of pure decay,
linearity in the cotangents, and planted mistakes that the differences
must catch."""
import numpy as np
import pytest

from oracle import backward as bw
from oracle.recurrence import kda_recurrent


def inputs(seed, T=13, H=2, dk=6, dv=5):
    r = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)   # noqa: E731
    d = {"q": unit(r.standard_normal((T, H, dk))), "k": unit(r.standard_normal((T, H, dk))),
         "v": r.standard_normal((T, H, dv)),
         "g": -5.0 / (1.0 + np.exp(-r.standard_normal((T, H, dk)))),
         "beta": 1.0 / (1.0 + np.exp(-r.standard_normal((T, H)))),
         "S0": r.standard_normal((H, dk, dv)) * 0.5}
    cot = {"dO": r.standard_normal((T, H, dv)), "dST": r.standard_normal((H, dk, dv))}
    return d, cot


def loss(d, cot):
    o, S = kda_recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    return float(np.sum(o * cot["dO"]) + np.sum(S * cot["dST"]))


def grads(d, cot, f=None):
    f = f or bw.kda_recurrent_vjp
    r = f(d["q"], d["k"], d["v"], d["g"], d["beta"], cot["dO"], d["S0"], cot["dST"])
    return dict(zip(("q", "k", "v", "g", "beta", "S0"), r))


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "S0"])
@pytest.mark.parametrize("seed", [0, 1])
def test_central_differences(name, seed):
    d, cot = inputs(seed)
    gr = grads(d, cot)
    r = np.random.default_rng(100 + seed)
    for _ in range(3):
        dirn = r.standard_normal(d[name].shape)
        eps = 1e-6
        dp = dict(d, **{name: d[name] + eps * dirn})
        dm = dict(d, **{name: d[name] - eps * dirn})
        fd = (loss(dp, cot) - loss(dm, cot)) / (2 * eps)
        an = float(np.sum(gr[name] * dirn))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (name, fd, an)


def test_pure_decay_closed_form():
    """beta = 0: the state only decays, so dk = dv = 0, and
    dq_t = (exp(sum_{s<=t} g_s) * S0) dO_t."""
    d, cot = inputs(3)
    d["beta"][:] = 0.0
    gr = grads(d, cot)
    assert np.all(gr["k"] == 0.0) and np.all(gr["v"] == 0.0)
    G = np.cumsum(d["g"], axis=0)
    for t in range(d["q"].shape[0]):
        St = np.exp(G[t])[:, :, None] * d["S0"]
        assert np.allclose(gr["q"][t], np.einsum("hij,hj->hi", St, cot["dO"][t]), atol=1e-12)


def test_linear_in_cotangents():
    d, c1 = inputs(4)
    _, c2 = inputs(5)
    mix = {key: 2.0 * c1[key] - 0.5 * c2[key] for key in c1}
    g1, g2, gm = grads(d, c1), grads(d, c2), grads(d, mix)
    for key in g1:
        assert np.allclose(gm[key], 2.0 * g1[key] - 0.5 * g2[key], atol=1e-10)


def test_varlen_is_per_sequence():
    d, cot = inputs(6, T=20)
    cu = np.array([0, 7, 7, 20])
    S0 = np.stack([d["S0"], d["S0"] * 0.3, -d["S0"]])
    dST = np.stack([cot["dST"], cot["dST"] * 2, cot["dST"] * -1])
    r = bw.kda_recurrent_vjp_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cot["dO"], cu,
                                    S0, dST)
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        one = bw.kda_recurrent_vjp(d["q"][a:b], d["k"][a:b], d["v"][a:b], d["g"][a:b],
                                   d["beta"][a:b], cot["dO"][a:b], S0[s], dST[s])
        for x, y in zip(r[:5], one[:5]):
            assert np.array_equal(x[a:b], y)
        assert np.array_equal(r[5][s], one[5])
    assert np.array_equal(r[5][1], dST[1])           # empty sequence: dS0 = dS_T


MUTANTS = {
    # decay gradient read off the undecayed state
    "dg_from_S_prev": ("dg[t] = np.sum(dSp * Sp[t], axis=-1)",
                       "dg[t] = np.sum(dSp * Sp[t] * np.exp(-g[t])[:, :, None], axis=-1)"),
    # the erase term's contribution to the state cotangent dropped
    "no_erase_in_dS": ("dSp = dS + k[t][:, :, None] * dw[:, None, :]", "dSp = dS"),
    # read gradient taken from the pre-update state
    "dq_from_Sprime": ('dq[t] = np.einsum("hij,hj->hi", Sn[t], dO[t])',
                       'dq[t] = np.einsum("hij,hj->hi", Sp[t], dO[t])'),
    # cotangent carried to the previous token without the decay
    "no_decay_carry": ("dS = dSp * np.exp(g[t])[:, :, None]", "dS = dSp"),
    # beta's gradient against v instead of the delta
    "dbeta_vs_v": ("db[t] = np.sum((v[t] - W[t]) * du, axis=-1)",
                   "db[t] = np.sum(v[t] * du, axis=-1)"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistakes_fail_the_differences(name):
    import inspect
    src = inspect.getsource(bw.kda_recurrent_vjp)
    old, new = MUTANTS[name]
    assert old in src
    ns = {"np": np, "Optional": bw.Optional, "Tuple": bw.Tuple}
    exec(src.replace(old, new), ns)
    mutant = ns["kda_recurrent_vjp"]
    d, cot = inputs(7)
    gr = grads(d, cot, mutant)
    r = np.random.default_rng(9)
    worst = 0.0
    for key in gr:
        dirn = r.standard_normal(d[key].shape)
        eps = 1e-6
        fd = (loss(dict(d, **{key: d[key] + eps * dirn}), cot)
              - loss(dict(d, **{key: d[key] - eps * dirn}), cot)) / (2 * eps)
        worst = max(worst, abs(fd - float(np.sum(gr[key] * dirn))) / max(1.0, abs(fd)))
    assert worst > 1e-4, name


# ---------------------------------------------------------------------------
# The plain-C VJP (oracle/kda_oracle.c, kda_oracle_vjp): central differences
# of the fp64 forward oracle at fp32-representable inputs (the C oracle reads
# fp32), and agreement with the NumPy VJP on packed batches.
# ---------------------------------------------------------------------------
def _f32_exact(d):
    return {key: np.asarray(x, np.float32).astype(np.float64) for key, x in d.items()}


def c_grads(d, cot):
    from oracle import clib
    T, H, _ = d["q"].shape
    r = clib.vjp(d["q"], d["k"], d["v"], d["g"], d["beta"], cot["dO"], np.array([0, T]),
                 d["S0"][None], cot["dST"][None])
    out = dict(zip(("q", "k", "v", "g", "beta"), r[:5]))
    out["S0"] = r[5][0]
    return out


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "S0"])
@pytest.mark.parametrize("seed", [0, 7])
def test_c_vjp_central_differences(name, seed):
    d, cot = inputs(seed)
    d, cot = _f32_exact(d), _f32_exact(cot)
    gr = c_grads(d, cot)
    r = np.random.default_rng(200 + seed)
    for _ in range(3):
        dirn = r.standard_normal(d[name].shape)
        eps = 1e-6
        dp = dict(d, **{name: d[name] + eps * dirn})
        dm = dict(d, **{name: d[name] - eps * dirn})
        fd = (loss(dp, cot) - loss(dm, cot)) / (2 * eps)
        an = float(np.sum(gr[name] * dirn))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (name, fd, an)


@pytest.mark.parametrize("with_state", [False, True])
def test_c_vjp_matches_numpy_on_packed_batches(with_state):
    from oracle import clib
    r = np.random.default_rng(11)
    cu = np.array([0, 1, 1, 17, 40, 41], np.int32)
    N, H, dk, dv = 41, 3, 8, 12
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)   # noqa: E731
    x = {"q": unit(r.standard_normal((N, H, dk))), "k": unit(r.standard_normal((N, H, dk))),
         "v": r.standard_normal((N, H, dv)),
         "g": -5.0 / (1.0 + np.exp(-r.standard_normal((N, H, dk)))),
         "beta": 1.0 / (1.0 + np.exp(-r.standard_normal((N, H)))),
         "dO": r.standard_normal((N, H, dv))}
    x = _f32_exact(x)
    S0 = dST = None
    if with_state:
        S0 = np.asarray(r.standard_normal((5, H, dk, dv)), np.float32).astype(np.float64)
        dST = np.asarray(r.standard_normal((5, H, dk, dv)), np.float32).astype(np.float64)
    a = clib.vjp(x["q"], x["k"], x["v"], x["g"], x["beta"], x["dO"], cu, S0, dST, threads=2)
    b = bw.kda_recurrent_vjp_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], x["dO"], cu,
                                    S0, dST)
    for got, ref in zip(a[:6], b):
        assert got.shape == ref.shape
        assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, float(np.max(np.abs(ref))))
