"""CPU pins of the speculative-decoding oracle (oracle/spec.py), against
facts from outside it: the independent C oracle run over the same token
streams as a prefill, the closed form of pure decay, and invariants of the
commit (nothing accepted leaves the state bit for bit; everything accepted
equals the whole stream)."""
import numpy as np
import pytest

from oracle import clib
from oracle.spec import kda_spec_commit, kda_spec_step, kda_spec_verify


def drafts(seed, N, K, H, dk, dv, beta_zero=False):
    r = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)   # noqa: E731
    d = {"q": unit(r.standard_normal((N, K, H, dk))), "k": unit(r.standard_normal((N, K, H, dk))),
         "v": r.standard_normal((N, K, H, dv)),
         "g": -5.0 / (1.0 + np.exp(-r.standard_normal((N, K, H, dk)))),
         "beta": 1.0 / (1.0 + np.exp(-r.standard_normal((N, K, H))))}
    if beta_zero:
        d["beta"][:] = 0.0
    d = {key: x.astype(np.float32) for key, x in d.items()}
    S = (r.standard_normal((N, H, dk, dv)) * 0.3).astype(np.float32)
    return d, S


def c_prefill(d, n, S, upto):
    """The C oracle on tokens 0..upto-1 of sequence n, all heads, from S[n]."""
    cu = np.array([0, upto], np.int32)
    o, ST, _ = clib.fwd(d["q"][n, :upto], d["k"][n, :upto], d["v"][n, :upto],
                        d["g"][n, :upto], d["beta"][n, :upto], cu, S[n][None])
    return o, ST[0]


def test_verify_equals_prefill_of_the_drafts():
    d, S = drafts(1, 3, 5, 2, 16, 8)
    o = kda_spec_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
    for n in range(3):
        o_ref, _ = c_prefill(d, n, S, 5)
        assert np.max(np.abs(o[n] - o_ref)) < 1e-12


def test_commit_equals_prefill_of_the_accepted_prefix():
    d, S = drafts(2, 4, 6, 2, 16, 8)
    acc = np.array([0, 1, 4, 6])
    S1 = kda_spec_commit(d["k"], d["v"], d["g"], d["beta"], acc, S)
    for n in range(4):
        if acc[n] == 0:
            assert np.array_equal(S1[n], S[n].astype(np.float64))
        else:
            _, ST = c_prefill(d, n, S, int(acc[n]))
            assert np.max(np.abs(S1[n] - ST)) < 1e-12


def test_commit_clamps_and_leaves_input_untouched():
    d, S = drafts(3, 2, 3, 1, 8, 8)
    S_copy = S.copy()
    S1 = kda_spec_commit(d["k"], d["v"], d["g"], d["beta"], np.array([-4, 99]), S)
    assert np.array_equal(S, S_copy)
    assert np.array_equal(S1[0], S[0].astype(np.float64))
    _, ST = c_prefill(d, 1, S, 3)
    assert np.max(np.abs(S1[1] - ST)) < 1e-12


def test_verify_pure_decay_closed_form():
    """beta = 0: o_j = S^T (exp(sum_{t<=j} g_t) * q_j), the state only decays."""
    d, S = drafts(4, 2, 4, 2, 8, 4, beta_zero=True)
    o = kda_spec_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
    G = np.cumsum(d["g"].astype(np.float64), axis=1)
    for n in range(2):
        for j in range(4):
            for h in range(2):
                ref = S[n, h].astype(np.float64).T @ (np.exp(G[n, j, h]) * d["q"][n, j, h])
                assert np.max(np.abs(o[n, j, h] - ref)) < 1e-12


@pytest.mark.parametrize("acc", [[0, 2], [3, 1]])
def test_step_is_commit_then_verify(acc):
    prev, S = drafts(5, 2, 3, 2, 16, 8)
    new, _ = drafts(6, 2, 4, 2, 16, 8)
    o, S1 = kda_spec_step(prev, np.array(acc), new, S)
    # the committed state is the prefill of the accepted prefix; the outputs
    # are the prefill of the new drafts from it
    for n in range(2):
        if acc[n]:
            _, ST = c_prefill(prev, n, S, acc[n])
        else:
            ST = S[n].astype(np.float64)
        assert np.max(np.abs(S1[n] - ST)) < 1e-12
        o_ref, _ = c_prefill(new, n, S1.astype(np.float32), 4)
        # S1 rounded to fp32 for the C oracle's input
        assert np.max(np.abs(o[n] - o_ref)) < 1e-5
