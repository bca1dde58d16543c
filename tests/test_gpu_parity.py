"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerance (max |x - ref| / rms(ref) over all compared elements): 1e-4 for
fp32 inputs, 2e-2 for bf16 inputs, on o and S_T.  For bf16-stored o the
storage rounding of each element (half a bf16 ulp of the exact value) is
allowed on top, see _gpu_util.err_bf16_out; the same kernels with an fp32 o
are held to the plain metric.
"""
import sys

import numpy as np
import pytest
import torch

from tests._gpu_util import err, err_bf16_out, random_batch, to_dev
from oracle import clib

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def kda():
    import gated_delta_rule_95_amd as m
    return m


def run_fwd(b, dtype, out_dtype=None, with_s0=True, packed=True):
    d = to_dev(b, dtype)
    o, ST = kda().kda_fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                  S0=d.get("s0") if with_s0 else None,
                                  cu_seqlens=d["cu_seqlens"] if packed else None,
                                  out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ST.cpu().numpy()


def oracle(b, with_s0=True):
    o, ST, _ = clib.fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], b["cu_seqlens"],
                        b.get("s0") if with_s0 else None, threads=16)
    return o, ST


# ---------------------------------------------------------------------------
def test_tiny_fp32_reference_workload():
    """B=1, H=1, T=64, d=16, fp32, S0 = 0: the tiny reference workload."""
    from synth import WORKLOADS, batch_inputs
    b = batch_inputs(WORKLOADS["tiny"])
    say("tiny fp32")
    o, ST = run_fwd(b, torch.float32, with_s0=False)
    o_ref, ST_ref = oracle(b, with_s0=False)
    assert err(o, o_ref) <= 1e-4
    assert err(ST, ST_ref) <= 1e-4


# every (d_k, d_v) pair the library builds is covered between the shapes
# here and the decode tests: narrow value blocks (d_v = 16, 32) with wide
# keys, the builder's two token-group layouts (four groups at d_k = 128,
# eight below), and the auxiliary-wave configuration (bf16, d_k = 128,
# d_v >= 64) with one and with two column blocks
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16), (16, 128),
                                   (128, 32), (64, 16), (128, 64)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_shapes_ragged(dk, dv, dtype):
    """Several chunks, a ragged tail, T=1 and an empty sequence, with S0."""
    lengths = [1, 0, 17, 100, 16, 47]
    b = random_batch(11 + dk + dv, lengths, H=3, dk=dk, dv=dv,
                     bf16=dtype == torch.bfloat16)
    say("shapes", dk, dv, dtype)
    o_ref, ST_ref = oracle(b)
    out = torch.float32
    o, ST = run_fwd(b, dtype, out_dtype=out)
    tol = TOL[dtype]
    assert err(o, o_ref) <= tol, err(o, o_ref)
    assert err(ST, ST_ref) <= tol, err(ST, ST_ref)
    # the empty sequence hands S0 through unchanged
    assert np.array_equal(ST[1], b["s0"][1])
    if dtype == torch.bfloat16:
        ob, STb = run_fwd(b, dtype, out_dtype=torch.bfloat16)
        assert err_bf16_out(ob, o_ref) <= tol
        # the bf16 store is the round-to-nearest-even of the fp32 result
        rn = torch.from_numpy(o).to(torch.bfloat16).float().numpy()
        assert np.array_equal(ob, rn)
        assert np.array_equal(STb, ST)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_no_s0_equal_lengths(dtype):
    """cu_seqlens = NULL: B equal-length sequences in [B, T, H, d] layout."""
    B, T, H, d = 3, 80, 2, 64
    b = random_batch(5, [T] * B, H=H, dk=d, dv=d, s0=False, bf16=dtype == torch.bfloat16)
    say("equal lengths", dtype)
    o_ref, ST_ref = oracle(b, with_s0=False)
    dd = to_dev(b, dtype)
    q = dd["q"].view(B, T, H, d)
    o, ST = kda().kda_fwd_chunked(q, dd["k"].view(B, T, H, d), dd["v"].view(B, T, H, d),
                                  dd["g"].view(B, T, H, d), dd["beta"].view(B, T, H),
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert o.shape == (B, T, H, d)
    assert err(o.reshape(B * T, H, d).cpu().numpy(), o_ref) <= TOL[dtype]
    assert err(ST.cpu().numpy(), ST_ref) <= TOL[dtype]


def test_decay_bound_stress():
    """g = -5 exactly on most channels (the tile's rescale factor is e^80),
    beta = 1 on some tokens, keys repeated inside tiles."""
    b = random_batch(77, [64, 33], H=2, dk=128, dv=128)
    b["g"][:] = -5.0
    b["g"][:, :, :8] = -0.01
    b["beta"][::5] = 1.0
    for base in range(0, 64, 16):
        b["k"][base + 8:base + 16] = b["k"][base:base + 8]
    say("decay bound stress")
    o_ref, ST_ref = oracle(b)
    o, ST = run_fwd(b, torch.bfloat16, out_dtype=torch.float32)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
    assert err(o, o_ref) <= 2e-2
    assert err(ST, ST_ref) <= 2e-2


def test_carry_over_segments():
    """fwd(x[0:T]) == fwd(x[T1:T], S0 = fwd(x[0:T1]).S_T), T1 not chunk-aligned."""
    T, T1, H, d = 200, 75, 2, 128
    b = random_batch(9, [T], H=H, dk=d, dv=d)
    say("carry over")
    d_ = to_dev(b, torch.bfloat16)
    m = kda()
    o_full, S_full = m.kda_fwd_chunked(d_["q"], d_["k"], d_["v"], d_["g"], d_["beta"],
                                       S0=d_["s0"], out_dtype=torch.float32)
    sl = lambda x, a, c: x[a:c].contiguous()
    o1, S1 = m.kda_fwd_chunked(*(sl(d_[x], 0, T1) for x in ("q", "k", "v", "g", "beta")),
                               S0=d_["s0"], out_dtype=torch.float32)
    o2, S2 = m.kda_fwd_chunked(*(sl(d_[x], T1, T) for x in ("q", "k", "v", "g", "beta")),
                               S0=S1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle(b)
    oc = torch.cat([o1, o2]).cpu().numpy()
    assert err(oc, o_ref) <= 2e-2
    assert err(S2.cpu().numpy(), S_ref) <= 2e-2
    assert err(o_full.cpu().numpy(), o_ref) <= 2e-2


def test_no_final_state():
    """S_T == NULL (output_final_state=False): o is still right and no state
    is written."""
    b = random_batch(13, [70, 16, 3], H=2, dk=128, dv=128)
    say("no final state")
    d = to_dev(b, torch.bfloat16)
    o, ST = kda().kda_fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["s0"],
                                  cu_seqlens=d["cu_seqlens"], out_dtype=torch.float32,
                                  output_final_state=False)
    torch.cuda.synchronize()
    assert ST is None
    o_ref, _ = oracle(b)
    assert err(o.cpu().numpy(), o_ref) <= 2e-2


def test_cu_seqlens_out_of_contract_stays_in_bounds():
    """A cu_seqlens past n_tokens (decreasing, [0, 300, 200] with 200 tokens)
    is clamped into [0, n_tokens]: nothing is read or written outside the
    buffers.  o sits at the start of a larger allocation whose tail is a
    guard that must come back untouched."""
    H, D, N = 2, 64, 200
    b = random_batch(17, [N], H=H, dk=D, dv=D)
    say("cu_seqlens clamp")
    d = to_dev(b, torch.bfloat16)
    cu = torch.tensor([0, 300, 200], dtype=torch.int32, device="cuda")
    S0 = torch.randn(2, H, D, D, device="cuda")
    big = torch.full((N + 64, H, D), 7.0, dtype=torch.float32, device="cuda")
    o = big[:N]
    _, ST = kda().kda_fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0,
                                  cu_seqlens=cu, out_dtype=torch.float32, o=o)
    torch.cuda.synchronize()
    assert torch.all(big[N:] == 7.0)
    assert torch.all(torch.isfinite(o)) and torch.all(torch.isfinite(ST))
    # after clamping, sequence 1 is empty: its state passes through
    assert torch.equal(ST[1], S0[1])


def test_deterministic():
    b = random_batch(3, [300, 5, 129], H=4, dk=128, dv=128)
    say("determinism")
    o1, S1 = run_fwd(b, torch.bfloat16)
    o2, S2 = run_fwd(b, torch.bfloat16)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


@pytest.mark.parametrize("n_seqs", [5, 64, 70, 128, 130])
def test_dispatch_order_keeps_state_slots(n_seqs):
    """Packed batches of up to 128 sequences are dealt to workgroups longest
    first (above 128 in index order).  Lengths increasing with the index, so
    the order reverses; every sequence has its own S0 and must read and write
    exactly its own state slot and token range.  70 sequences cover the
    second rank register (sequences 64 and up), 130 the index order."""
    lengths = [1 + (3 * i) % 37 + i // 4 for i in range(n_seqs)]
    lengths[n_seqs // 2] = 0
    b = random_batch(41 + n_seqs, lengths, H=2, dk=32, dv=32, bf16=False)
    say("dispatch order", n_seqs)
    o_ref, ST_ref = oracle(b)
    o, ST = run_fwd(b, torch.float32, out_dtype=torch.float32)
    assert err(o, o_ref) <= 1e-4, err(o, o_ref)
    for n in range(n_seqs):
        assert err(ST[n], ST_ref[n]) <= 1e-4, (n, err(ST[n], ST_ref[n]))
    assert np.array_equal(ST[n_seqs // 2], b["s0"][n_seqs // 2])


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 128), (32, 64), (64, 128), (128, 128), (128, 32)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_small(dk, dv, dtype):
    from oracle.recurrence import kda_decode_step as ref_step
    r = np.random.default_rng(dk * 1000 + dv)
    N, H = 5, 3
    b = random_batch(dk + dv, [1] * N, H=H, dk=dk, dv=dv, bf16=dtype == torch.bfloat16)
    S = (r.standard_normal((N, H, dk, dv)) * 0.05).astype(np.float32)
    say("decode", dk, dv, dtype)
    o_ref, S_ref = ref_step(b["q"], b["k"], b["v"], b["g"], b["beta"], S)
    d = to_dev(b, dtype)
    Sd = torch.from_numpy(S).cuda()
    o = kda().kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], Sd,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert err(o.cpu().numpy(), o_ref) <= TOL[dtype]
    assert err(Sd.cpu().numpy(), S_ref) <= TOL[dtype]


def test_decode_chain_equals_prefill():
    """T decode steps from S0 give the prefill's o and S_T (same inputs)."""
    T, H, d = 20, 2, 128
    b = random_batch(21, [T], H=H, dk=d, dv=d)
    say("decode chain")
    dd = to_dev(b, torch.bfloat16)
    m = kda()
    o_pf, S_pf = m.kda_fwd_chunked(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"],
                                   S0=dd["s0"], out_dtype=torch.float32)
    S = dd["s0"].clone()
    outs = []
    for t in range(T):
        sl = lambda x: x[t:t + 1].contiguous()
        outs.append(m.kda_decode_step(sl(dd["q"]), sl(dd["k"]), sl(dd["v"]), sl(dd["g"]),
                                      sl(dd["beta"]), S, out_dtype=torch.float32))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle(b)
    assert err(torch.cat(outs).cpu().numpy(), o_ref) <= 1e-4   # fp32 state math
    assert err(S.cpu().numpy(), S_ref) <= 1e-4
    assert err(o_pf.cpu().numpy(), o_ref) <= 2e-2
    assert err(S_pf.cpu().numpy(), S_ref) <= 2e-2


# ---------------------------------------------------------------------------
# errors surface as exceptions, never as silent results
# ---------------------------------------------------------------------------
def test_binding_rejects_bad_arguments():
    m = kda()
    q = torch.zeros(4, 2, 48, device="cuda", dtype=torch.bfloat16)
    g = torch.zeros(4, 2, 48, device="cuda")
    beta = torch.zeros(4, 2, device="cuda")
    with pytest.raises(m.KDAError) as ei:
        m.kda_fwd_chunked(q, q, q, g, beta)
    assert ei.value.status == 2          # KDA_ERR_UNSUPPORTED (d = 48)
    q16 = torch.zeros(4, 2, 16, device="cuda", dtype=torch.float16)
    with pytest.raises(TypeError):
        m.kda_fwd_chunked(q16, q16, q16, g[..., :16].contiguous(), beta)
