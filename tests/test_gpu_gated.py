"""GPU parity of kda_fwd_chunked_gated (gate, beta and q/k L2 normalisation
fused into the prefill) through the C ABI against the fp64 oracle
(oracle/prologue.py, then the recurrence).

Tolerance as elsewhere: max |x - ref| / rms(ref) <= 1e-4 (fp32 inputs) or
2e-2 (bf16 inputs; bf16 o with the half-ulp storage allowance)."""
import sys
import time

import numpy as np
import pytest
import torch

from oracle import clib
from oracle.prologue import kda_prologue
from synth import WORKLOADS, batch_inputs, round_bf16, seq_lengths
from tests._gpu_util import err, err_bf16_out, half_ulp_bf16

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def kda():
    import gated_delta_rule_95_amd as m
    return m


def raw_batch(seed, lengths, H, dk, dv, bf16, s0=True):
    r = np.random.default_rng(seed)
    lengths = np.asarray(lengths, np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = int(cu[-1])
    # unnormalised q, k with token scales from 0.05 to 20
    scale = np.exp(r.uniform(np.log(0.05), np.log(20.0), (N, H, 1))).astype(np.float32)
    d = {"q": r.standard_normal((N, H, dk)).astype(np.float32) * scale,
         "k": r.standard_normal((N, H, dk)).astype(np.float32) * scale[:, ::-1],
         "v": r.standard_normal((N, H, dv)).astype(np.float32),
         "z": (r.standard_normal((N, H, dk)) * 1.5).astype(np.float32),
         "b": r.standard_normal((N, H)).astype(np.float32),
         "A_log": (r.standard_normal(H) * 0.5).astype(np.float32),
         "cu_seqlens": cu}
    if bf16:
        for key in ("q", "k", "v", "z", "b"):
            d[key] = round_bf16(d[key])
    if s0:
        d["s0"] = (r.standard_normal((len(lengths), H, dk, dv)) * 0.3).astype(np.float32)
    return d


def oracle(d, s0=True):
    """fp64 prologue, then the C recurrence on its outputs (rounded to fp32:
    the C oracle reads fp32; that rounding is far below either bar)."""
    qn, kn, g, beta = kda_prologue(d["q"], d["k"], d["z"], d["A_log"], d["b"])
    f = lambda x: np.asarray(x, np.float32)               # noqa: E731
    o, S, _ = clib.fwd(f(qn), f(kn), d["v"], f(g), f(beta), d["cu_seqlens"],
                       d.get("s0") if s0 else None)
    return o, S


def to_dev(d, dtype):
    t = {key: torch.from_numpy(d[key]).cuda().to(dtype) for key in ("q", "k", "v", "z", "b")}
    t["A_log"] = torch.from_numpy(d["A_log"]).cuda()
    t["cu_seqlens"] = torch.from_numpy(d["cu_seqlens"]).cuda()
    if "s0" in d:
        t["s0"] = torch.from_numpy(d["s0"]).cuda()
    return t


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16),
                                   (16, 128), (128, 64)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gated_shapes_ragged(dk, dv, dtype):
    """Ragged lengths (1, 0, 17, 100, 16, 47): the padded tokens of every
    chunk tail must stay identity transitions although z = 0 there."""
    bf = dtype == torch.bfloat16
    d = raw_batch(dk * 3 + dv, [1, 0, 17, 100, 16, 47], 3, dk, dv, bf)
    say("gated", dk, dv, dtype)
    o_ref, S_ref = oracle(d)
    t = to_dev(d, dtype)
    o, S = kda().kda_fwd_chunked_gated(t["q"], t["k"], t["v"], t["z"], t["A_log"], t["b"],
                                       S0=t["s0"], cu_seqlens=t["cu_seqlens"],
                                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    tol = 2e-2 if bf else 1e-4
    eo, es = err(o.cpu().numpy(), o_ref), err(S.cpu().numpy(), S_ref)
    say(f"  o {eo:.2e} S_T {es:.2e}")
    assert eo <= tol and es <= tol
    assert np.array_equal(S.cpu().numpy()[1], d["s0"][1])      # empty sequence


def test_gated_matches_plain_entry_on_host_prologue():
    """The fused prologue against kda_fwd_chunked fed with the prologue's
    outputs computed on the host in fp32."""
    d = raw_batch(5, [300, 77], 4, 128, 128, False)
    qn, kn, g, beta = (np.asarray(x, np.float32) for x in
                       kda_prologue(d["q"], d["k"], d["z"], d["A_log"], d["b"]))
    t = to_dev(d, torch.float32)
    m = kda()
    o1, S1 = m.kda_fwd_chunked_gated(t["q"], t["k"], t["v"], t["z"], t["A_log"], t["b"],
                                     S0=t["s0"], cu_seqlens=t["cu_seqlens"])
    c = lambda x: torch.from_numpy(x).cuda()               # noqa: E731
    o2, S2 = m.kda_fwd_chunked(c(qn), c(kn), t["v"], c(g), c(beta), S0=t["s0"],
                               cu_seqlens=t["cu_seqlens"])
    torch.cuda.synchronize()
    assert err(o1.cpu().numpy(), o2.cpu().numpy().astype(np.float64)) <= 1e-4
    assert err(S1.cpu().numpy(), S2.cpu().numpy().astype(np.float64)) <= 1e-4


def test_gated_split_path():
    """Few heads, one long sequence: the sequence-split path with the fused
    prologue, against the oracle and the single pass."""
    T, H, D = 4096, 4, 128
    m = kda()
    assert m.kda_fwd_workspace_bytes(1, T, H, D, D, torch.bfloat16) > 0
    d = raw_batch(9, [T], H, D, D, True)
    o_ref, S_ref = oracle(d)
    t = to_dev(d, torch.bfloat16)
    outs = []
    for ws in (True, False):
        o, S = m.kda_fwd_chunked_gated(t["q"], t["k"], t["v"], t["z"], t["A_log"], t["b"],
                                       S0=t["s0"], workspace=ws)
        outs.append((o.float().cpu().numpy(), S.cpu().numpy()))
    torch.cuda.synchronize()
    for (o, S), tag in zip(outs, ("split", "single")):
        eo, es = err_bf16_out(o, o_ref), err(S, S_ref)
        say(f"  gated {tag}: o {eo:.2e} S_T {es:.2e}")
        assert eo <= 2e-2 and es <= 2e-2


@pytest.mark.timeout(600)
def test_gated_prefill_workload_all_chains():
    """The prefill workload's shape (4 x 4096 tokens, H = 32, d = 128, bf16)
    from its raw pre-activation draws (A_log = 0), as bench.py runs it; every
    (sequence, head) chain against the oracle."""
    wl = WORKLOADS["prefill"]
    L = seq_lengths(wl)
    b = batch_inputs(wl, raw=True)
    B, T, H, D = len(L), wl.seqlen, wl.H, wl.dk
    say("gated prefill workload")
    t = {key: torch.from_numpy(b[key]).cuda().to(torch.bfloat16) for key in ("q", "k", "v", "z", "b")}
    A_log = torch.zeros(H, device="cuda")
    shp = (B, T, H)
    o = torch.full((B, T, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    S_T = torch.full((B, H, D, D), float("nan"), device="cuda")
    kda().kda_fwd_chunked_gated(t["q"].view(*shp, D), t["k"].view(*shp, D),
                                t["v"].view(*shp, D), t["z"].view(*shp, D), A_log,
                                t["b"].view(*shp), o=o, S_T=S_T)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().reshape(B * T, H, D)
    S_T = S_T.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S_T))
    t0 = time.perf_counter()
    d = {"q": b["q"], "k": b["k"], "v": b["v"], "z": b["z"], "b": b["b"],
         "A_log": np.zeros(H, np.float32), "cu_seqlens": b["cu_seqlens"]}
    o_ref, S_ref = oracle(d, s0=False)
    dev_o = np.maximum(np.abs(o - o_ref) - half_ulp_bf16(o_ref), 0.0)
    eo = float(dev_o.max()) / float(np.sqrt(np.mean(o_ref ** 2)))
    es = err(S_T, S_ref)
    say(f"  all {B} x {H} chains: o {eo:.2e} S_T {es:.2e} (oracle {time.perf_counter() - t0:.1f}s)")
    assert eo <= 2e-2 and es <= 2e-2
