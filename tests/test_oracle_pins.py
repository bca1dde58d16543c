"""CPU tests: every formulation of the oracle against the pins in _pins.py,
plus agreement between the C and NumPy recurrences on packed varlen
batches, the chunked form at the decay bound, and the decode step."""
import numpy as np
import pytest

from tests import _pins
from oracle import clib
from oracle.recurrence import kda_recurrent, kda_recurrent_varlen, kda_decode_step
from oracle.chunked import kda_chunked
from oracle.transition import kda_transition_bruteforce


def impl_numpy(q, k, v, g, beta, S0):
    o, S = kda_recurrent(np.asarray(q)[:, None], np.asarray(k)[:, None], np.asarray(v)[:, None],
                         np.asarray(g)[:, None], np.asarray(beta)[:, None],
                         None if S0 is None else np.asarray(S0)[None])
    return o[:, 0], S[0]


def impl_chunk(C):
    def f(q, k, v, g, beta, S0):
        return kda_chunked(q, k, v, g, beta, S0, chunk=C)
    return f


IMPLS = {
    "numpy": impl_numpy,
    "chunked16": impl_chunk(16),
    "chunked32": impl_chunk(32),
    "chunked64": impl_chunk(64),
    "bruteforce": kda_transition_bruteforce,
}


@pytest.mark.parametrize("pin", _pins.ALL_PINS, ids=lambda p: p.__name__)
@pytest.mark.parametrize("name", list(IMPLS))
def test_pin(name, pin):
    if name == "bruteforce" and pin is _pins.pin_bruteforce:
        pytest.skip("brute force is the reference of this pin")
    assert pin(IMPLS[name])


@pytest.mark.parametrize("pin", [_pins.pin_pure_decay, _pins.pin_hand_example,
                                 _pins.pin_linear_attention, _pins.pin_onehot_overwrite,
                                 _pins.pin_retrieval, _pins.pin_carry_over],
                         ids=lambda p: p.__name__)
def test_c_oracle_pins_fp32_exact(pin):
    """The C oracle reads fp32 inputs: pin it on fp32-rounded inputs (the
    closed forms see the same rounded values); unit keys and orthonormal
    bases are then only unit/orthonormal to fp32 precision, hence 2e-6."""
    with _pins.fp32_inputs():
        assert pin(clib.head)


@pytest.mark.parametrize("seed,dk,dv", [(1, 16, 16), (2, 8, 5), (3, 32, 16)])
def test_c_matches_numpy_varlen(seed, dk, dv):
    r = np.random.default_rng(seed)
    lens = np.array([37, 0, 1, 64, 16, 5])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N, H = int(cu[-1]), 3
    q = r.standard_normal((N, H, dk)).astype(np.float32)
    k = (r.standard_normal((N, H, dk)) / np.sqrt(dk)).astype(np.float32)
    v = r.standard_normal((N, H, dv)).astype(np.float32)
    g = r.uniform(-5, 0, (N, H, dk)).astype(np.float32)
    beta = r.uniform(0, 1, (N, H)).astype(np.float32)
    S0 = r.standard_normal((len(lens), H, dk, dv)).astype(np.float32)
    o1, S1 = kda_recurrent_varlen(q, k, v, g, beta, cu, S0)
    o2, S2, used = clib.fwd(q, k, v, g, beta, cu, S0, threads=4)
    assert used >= 1
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(S1 - S2)) < 1e-12
    # an empty sequence hands its S0 straight through
    assert np.array_equal(S2[1], S0[1].astype(np.float64))
    # packed run == separate runs (sequences never interact)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        o3, S3 = kda_recurrent(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], S0[n])
        assert np.max(np.abs(o3 - o1[a:b]), initial=0) < 1e-12
        assert np.max(np.abs(S3 - S1[n])) < 1e-12


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 100])
def test_chunked_at_decay_bound(C, T):
    """g = -5 exactly (the lower bound) puts a 16-token tile's cumulative
    log-decay at -80; the re-referenced chunk form must still match."""
    r = np.random.default_rng(T * 7 + C)
    dk, dv = 8, 6
    q = _pins._unit(r.standard_normal((T, dk)))
    k = _pins._unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    g = np.full((T, dk), -5.0)
    g[:, 0] = -1e-3                                   # one long-memory channel
    beta = r.uniform(0, 1, T)
    S0 = r.standard_normal((dk, dv))
    o1, S1 = impl_numpy(q, k, v, g, beta, S0)
    o2, S2 = kda_chunked(q, k, v, g, beta, S0, chunk=C)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(S2))
    assert np.max(np.abs(o1 - o2)) < 1e-10
    assert np.max(np.abs(S1 - S2)) < 1e-10


def test_tile_bound_fits_bf16_and_fp32():
    """With g >= -5 a 16-token tile's cumulative log-decay is >= -80: the
    rescale factor e^80 is below the largest bf16 / fp32 value and e^-80 is
    above the smallest normal fp32, so both directions stay finite."""
    bf16_max = (2 - 2 ** -7) * 2.0 ** 127
    fp32_min_normal = 2.0 ** -126
    assert 16 * 5 == 80
    assert np.exp(80.0) < bf16_max
    assert np.exp(-80.0) > fp32_min_normal
    # 17 tokens would still fit, 18 would not
    assert np.exp(17 * 5.0) < bf16_max < np.exp(18 * 5.0)


def test_decode_chain_equals_prefill():
    """T successive single-token steps give the prefill's o and S_T."""
    r = np.random.default_rng(5)
    T, N, H, dk, dv = 9, 2, 3, 6, 4
    q = r.standard_normal((T, N, H, dk))
    k = _pins._unit(r.standard_normal((T, N, H, dk)))
    v = r.standard_normal((T, N, H, dv))
    g = r.uniform(-5, 0, (T, N, H, dk))
    beta = r.uniform(0, 1, (T, N, H))
    S = r.standard_normal((N, H, dk, dv))
    S0 = S.copy()
    outs = []
    for t in range(T):
        o, S = kda_decode_step(q[t], k[t], v[t], g[t], beta[t], S)
        outs.append(o)
    for n in range(N):
        o_ref, S_ref = kda_recurrent(q[:, n], k[:, n], v[:, n], g[:, n], beta[:, n], S0[n])
        assert np.max(np.abs(np.stack(outs)[:, n] - o_ref)) < 1e-12
        assert np.max(np.abs(S[n] - S_ref)) < 1e-12


def test_state_size_independent_of_T():
    """The state handed back is d_k x d_v per (sequence, head) whatever T."""
    shapes = set()
    for T in (1, 64, 1000):
        r = np.random.default_rng(T)
        q = r.standard_normal((T, 2, 8)).astype(np.float32)
        _, ST, _ = clib.fwd(q, q, r.standard_normal((T, 2, 4)), -np.ones((T, 2, 8)),
                            np.ones((T, 2)) * 0.5, np.array([0, T], np.int32), want_o=False)
        shapes.add(ST.shape)
    assert shapes == {(1, 2, 8, 4)}
