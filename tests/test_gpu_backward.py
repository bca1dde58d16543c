"""GPU parity of the chunked backward (kda_bwd_chunked) through the C ABI
against the fp64 reverse-mode oracle (oracle/backward.py; at full size its
plain-C counterpart, oracle/kda_oracle.c).

Every gradient (dq, dk, dv, dg, dbeta, dS0) is compared element by element:
max |x - ref| / rms(ref) <= 1e-4 for fp32 inputs and 2e-2 for bf16 inputs
(the forward's bars; the backward computes in fp32 either way).
"""
import sys

import numpy as np
import pytest
import torch

from oracle.backward import kda_recurrent_vjp_varlen
from synth import round_bf16
from tests._gpu_util import err, random_batch

pytestmark = pytest.mark.gpu
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def kda():
    import gated_delta_rule_95_amd as m
    return m


def cotangents(seed, b, bf16, with_dST=True):
    r = np.random.default_rng(seed)
    N, H, _ = b["q"].shape
    dv = b["v"].shape[-1]
    dO = r.standard_normal((N, H, dv)).astype(np.float32)
    if bf16:
        dO = round_bf16(dO)
    ns = len(b["cu_seqlens"]) - 1
    dST = (r.standard_normal((ns, H, b["q"].shape[-1], dv)).astype(np.float32)
           if with_dST else None)
    return dO, dST


def run(b, dO, dST, dtype, packed=True, with_s0=True):
    """packed: [N, H, d] with cu_seqlens; otherwise the equal-length batch as
    [B, T, H, d] with cu_seqlens = NULL (gradients flattened back to N)."""
    cu = b["cu_seqlens"]
    B, N = len(cu) - 1, int(cu[-1])
    lead = (N,) if packed else (B, N // B)

    def dev(x):
        x = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        return x.view(lead + x.shape[1:]) if x.shape[0] == N else x

    t = {key: dev(b[key]).to(dtype) for key in ("q", "k", "v")}
    out = kda().kda_bwd_chunked(t["q"], t["k"], t["v"], dev(b["g"]), dev(b["beta"]),
                                dev(dO).to(dtype), S0=dev(b["s0"]) if with_s0 else None,
                                dS_T=None if dST is None else dev(dST),
                                cu_seqlens=dev(cu) if packed else None)
    torch.cuda.synchronize()
    return [x.cpu().numpy().reshape((N,) + tuple(x.shape[len(lead):])) if i < 5
            else x.cpu().numpy() for i, x in enumerate(out)]


def oracle(b, dO, dST, with_s0=True):
    return kda_recurrent_vjp_varlen(b["q"], b["k"], b["v"], b["g"], b["beta"], dO,
                                    b["cu_seqlens"], b["s0"] if with_s0 else None, dST)


def compare(got, ref, tol, tag):
    """Every gradient's error is printed before any is asserted."""
    errs = {}
    for name, x, y in zip(NAMES, got, ref):
        errs[name] = err(x, y) if np.all(np.isfinite(x)) else float("inf")
        say(f"  {tag} {name}: {errs[name]:.2e}")
    bad = {k: e for k, e in errs.items() if not e <= tol}
    assert not bad, bad
    return max(errs.values())


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16),
                                   (16, 128), (128, 64), (32, 32)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_bwd_shapes_ragged(dk, dv, dtype):
    """Packed lengths 1, 0, 17, 100, 16, 47: several chunks, ragged tails, a
    one-token and an empty sequence, with S0 and dS_T."""
    bf = dtype == torch.bfloat16
    b = random_batch(31 + dk + dv, [1, 0, 17, 100, 16, 47], H=3, dk=dk, dv=dv, bf16=bf)
    dO, dST = cotangents(7 + dk, b, bf)
    say("bwd", dk, dv, dtype)
    got = run(b, dO, dST, dtype)
    ref = oracle(b, dO, dST)
    compare(got, ref, 2e-2 if bf else 1e-4, f"{dk}x{dv}")
    # the empty sequence passes dS_T through to dS0
    assert np.array_equal(got[5][1], dST[1])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_bwd_equal_lengths_no_final_cotangent(dtype):
    """cu_seqlens = NULL ([B, T, H, d] layout), dS_T = NULL, no S0."""
    bf = dtype == torch.bfloat16
    B, T, H, d = 3, 80, 2, 64
    b = random_batch(5, [T] * B, H=H, dk=d, dv=d, s0=False, bf16=bf)
    dO, _ = cotangents(6, b, bf, with_dST=False)
    got = run(b, dO, None, dtype, packed=False, with_s0=False)
    ref = oracle(b, dO, None, with_s0=False)
    compare(got, ref, 2e-2 if bf else 1e-4, "equal lengths")


@pytest.mark.timeout(300)
def test_bwd_longer_sequences():
    """Two sequences of 700 and 1030 tokens, four heads, d = 128, bf16."""
    b = random_batch(9, [700, 1030], H=4, dk=128, dv=128, bf16=True)
    dO, dST = cotangents(10, b, True)
    got = run(b, dO, dST, torch.bfloat16)
    ref = oracle(b, dO, dST)
    compare(got, ref, 2e-2, "long")


def test_bwd_rejects_small_workspace():
    b = random_batch(3, [40], H=1, dk=16, dv=16)
    m = kda()
    need = m._lib.load().kda_bwd_workspace_bytes(1, 40, 1, 16, 16)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    t = {key: torch.from_numpy(b[key]).cuda() for key in ("q", "k", "v", "g", "beta")}
    with pytest.raises(m.KDAError):
        m.kda_bwd_chunked(t["q"], t["k"], t["v"], t["g"], t["beta"], t["v"].clone(),
                          workspace=ws)


@pytest.mark.timeout(600)
def test_bwd_prefill_workload_all_chains():
    """The prefill workload's shape (4 x 4096 tokens, H = 32, d = 128, bf16)
    with random cotangents: every gradient of every (sequence, head) chain
    against the plain-C fp64 oracle (OpenMP over chains), each chain's
    errors taken against that chain's own scale."""
    from oracle import clib
    from synth import WORKLOADS, batch_inputs
    wl = WORKLOADS["prefill"]
    b = batch_inputs(wl)
    cu = b["cu_seqlens"]
    ns, H = len(cu) - 1, wl.H
    dO, dST = cotangents(21, b, True)
    say("bwd prefill workload")
    got = run(b, dO, dST, torch.bfloat16, with_s0="s0" in b)
    for x in got:
        assert np.all(np.isfinite(x))
    say("bwd prefill workload: C oracle")
    ref = clib.vjp(b["q"], b["k"], b["v"], b["g"], b["beta"], dO, cu, b.get("s0"), dST,
                   threads=16)[:6]
    worst = {name: 0.0 for name in NAMES}
    for s in range(ns):
        lo, hi = int(cu[s]), int(cu[s + 1])
        for h in range(H):
            sl = lambda x: x[lo:hi, h]                         # noqa: E731
            mine = [sl(x) for x in got[:5]] + [got[5][s, h]]
            want = [sl(x) for x in ref[:5]] + [ref[5][s, h]]
            for name, x, y in zip(NAMES, mine, want):
                worst[name] = max(worst[name], err(x, y))
    say("  worst over the chains:", {k: f"{e:.2e}" for k, e in worst.items()})
    bad = {k: e for k, e in worst.items() if not e <= 2e-2}
    assert not bad, bad
