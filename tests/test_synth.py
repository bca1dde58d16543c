"""CPU tests of the seeded input generator (shared by the oracle and the HIP
path): reproducibility, value ranges and the stress structure."""
import numpy as np

from synth import (WORKLOADS, batch_inputs, bf16_bits, bf16_bits_to_f32, head_inputs,
                   round_bf16, seq_lengths, decode_head_inputs)


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38, 1e-40], np.float32)
    r = round_bf16(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                       # tie -> even mantissa
    assert r[2] == np.float32(1.0 + 2 ** -6)  # tie -> even (up)
    assert r[3] == -2.5
    assert np.array_equal(bf16_bits_to_f32(bf16_bits(r)), r)


def test_reproducible_and_head_local():
    wl = WORKLOADS["prefill"]
    a = head_inputs(wl, 2, 5, 100)
    b = head_inputs(wl, 2, 5, 100)
    c = head_inputs(wl, 2, 6, 100)
    for key in a:
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["q"], c["q"])


def test_value_ranges():
    wl = WORKLOADS["prefill"]
    d = head_inputs(wl, 0, 0, 512)
    assert np.all(d["g"] < 0) and np.all(d["g"] >= -5)
    assert np.all((d["beta"] > 0) & (d["beta"] < 1))
    n = np.linalg.norm(d["k"], axis=1)
    assert np.all(np.abs(n - 1) < 2 ** -7)
    assert np.array_equal(round_bf16(d["q"]), d["q"])       # bf16-exact
    tiny = head_inputs(WORKLOADS["tiny"], 0, 0, 64)
    assert tiny["q"].dtype == np.float32 and tiny["q"].shape == (64, 16)


def test_stress_structure():
    wl = WORKLOADS["varlen"]
    L = seq_lengths(wl)
    assert len(L) == 64 and L.min() >= 128 and L.max() <= 32768
    d0 = head_inputs(wl, 0, 0, 40)       # near-bound head
    d1 = head_inputs(wl, 0, 20, 40)      # ordinary head
    assert np.all(d0["g"] >= -5) and np.all(d0["g"] <= -4.9)
    assert d1["g"].max() > -4.9
    for base in (0, 16):
        assert np.array_equal(d0["k"][base + 8:base + 16], d0["k"][base:base + 8])
    # beta = 1 on the same positions for every head
    m0, m1 = d0["beta"] == 1.0, d1["beta"] == 1.0
    assert np.array_equal(m0, m1)


def test_batch_layout():
    wl = WORKLOADS["tiny"]
    b = batch_inputs(wl)
    assert b["q"].shape == (64, 1, 16) and b["beta"].shape == (64, 1)
    assert list(b["cu_seqlens"]) == [0, 64]
    d = head_inputs(wl, 0, 0, 64)
    assert np.array_equal(b["k"][:, 0], d["k"])


def test_decode_inputs():
    wl = WORKLOADS["decode"]
    d = decode_head_inputs(wl, 3, 7)
    assert d["S"].shape == (128, 128) and d["q"].shape == (128,)
    assert 0.04 < d["S"].std() < 0.06


def test_raw_draws_are_the_prologue_inputs():
    """raw=True gives the draws behind the regular inputs: normalising q, k
    and mapping z, b through the gate and sigmoid (on the host, here) gives
    back the regular fp32 workload inputs before bf16 rounding."""
    wl = WORKLOADS["long_prefill"]
    r = head_inputs(wl, 0, 3, 50, raw=True)
    d = head_inputs(wl, 0, 3, 50)
    assert set(r) == {"q", "k", "v", "z", "b", "s0"}
    assert np.array_equal(r["v"], d["v"]) and np.array_equal(r["s0"], d["s0"])
    g = -5.0 / (1.0 + np.exp(-r["z"].astype(np.float64)))
    assert np.max(np.abs(g - d["g"])) < 0.05          # z is bf16-rounded in raw mode
    qn = r["q"] / np.linalg.norm(r["q"], axis=1, keepdims=True)
    assert np.max(np.abs(qn - d["q"])) < 2e-2
    b = batch_inputs(WORKLOADS["prefill"], raw=True, seqs=range(1, 2))
    assert set(b) >= {"q", "k", "v", "z", "b", "cu_seqlens"}
