"""The pins must be able to fail.  Each mutant below is a copy of the token
recurrence with one plausible mistake planted in it (on the CPU, in this
test only); every mutant has to be rejected by at least one pin, while the
unmutated copy passes them all."""
import numpy as np
import pytest

from tests import _pins


def recurrence(q, k, v, g, beta, S0, m=""):
    q, k, v, g, beta = (np.asarray(x, np.float64) for x in (q, k, v, g, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64, copy=True)
    o = np.zeros((T, dv))
    for t in range(T):
        gt = g[t - 1] if (m == "decay_off_by_one" and t > 0) else g[t]
        a = np.exp(-gt) if m == "exp_sign" else np.exp(gt)
        Sold = S.copy()
        if m == "no_decay":
            pass
        elif m == "decay_columns":
            S = S * a[None, :dv] if dk == dv else S * a[:, None] * 0.999
        else:
            S = S * a[:, None]
        ref = Sold if m == "erase_before_decay" else S
        w = ref @ k[t] if (m == "transposed_delta" and dk == dv) else ref.T @ k[t]
        if m == "beta_on_v_only":
            u = beta[t] * v[t] - w
        elif m == "no_beta":
            u = v[t] - w
        else:
            u = beta[t] * (v[t] - w)
        if m == "erase_before_decay":
            S = S + np.outer(k[t], u)
        elif m == "sign_flip":
            S = S - np.outer(k[t], u)
        elif m == "write_q":
            S = S + np.outer(q[t], u)
        else:
            S = S + np.outer(k[t], u)
        if m == "read_before_update":
            o[t] = Sold.T @ q[t]
        elif m == "read_decayed_only":
            o[t] = (S - np.outer(k[t], u)).T @ q[t]
        elif m == "transposed_read" and dk == dv:
            o[t] = S @ q[t]
        elif m == "attention_scale":
            o[t] = S.T @ q[t] / np.sqrt(dk)
        else:
            o[t] = S.T @ q[t]
    return o, S


MUTANTS = ["decay_off_by_one", "exp_sign", "no_decay", "decay_columns",
           "erase_before_decay", "transposed_delta", "beta_on_v_only", "no_beta",
           "sign_flip", "write_q", "read_before_update", "read_decayed_only",
           "transposed_read", "attention_scale"]


def _passes(impl, pin):
    try:
        with np.errstate(all="ignore"):
            return bool(pin(impl))
    except Exception:
        return False


def test_unmutated_copy_passes_all_pins():
    impl = lambda *a: recurrence(*a)
    for pin in _pins.ALL_PINS:
        assert _passes(impl, pin), pin.__name__


@pytest.mark.parametrize("mutant", MUTANTS)
def test_mutant_is_caught(mutant):
    impl = lambda *a: recurrence(*a, m=mutant)
    caught = [p.__name__ for p in _pins.ALL_PINS if not _passes(impl, p)]
    assert caught, f"no pin rejects mutant {mutant}"
