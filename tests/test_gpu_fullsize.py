"""GPU parity at the full workload sizes, in the launch configuration the
bench times, on (sequence, head) chains sampled from the whole run.

Each test runs one whole workload through the C ABI, then regenerates the
sampled chains on the host from the same seeds (synth.head_inputs) and runs
the fp64 oracle on exactly those chains.  Tolerance as in test_gpu_parity:
max |x - ref| / rms(ref) <= 2e-2 on o (bf16-stored, half-ulp storage
allowance) and on S_T.  Every output element is also checked to be finite.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import clib
from oracle.recurrence import kda_decode_step as ref_decode
from synth import WORKLOADS, batch_inputs, decode_batch_inputs, head_inputs
from tests._gpu_util import err, err_bf16_out, to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def kda():
    import gated_delta_rule_95_amd as m
    return m


def reference(wl, n, h, T):
    d = head_inputs(wl, n, h, T)
    return clib.head(d["q"], d["k"], d["v"], d["g"], d["beta"], d.get("s0"))


def check_chain(wl, n, h, T, o_gpu, S_gpu, tag, ref=None):
    o_ref, S_ref = ref if ref is not None else reference(wl, n, h, T)
    eo, es = err_bf16_out(o_gpu, o_ref), err(S_gpu, S_ref)
    say(f"  {tag} seq {n} head {h} T {T}: o {eo:.2e}  S_T {es:.2e}")
    assert eo <= TOL and es <= TOL


def test_prefill_workload_sampled():
    """4 x 4096 tokens, H = 32, d = 128, bf16, S0 = 0, equal lengths
    (cu_seqlens = NULL, [B, T, H, d] layout), exactly as bench.py runs it."""
    wl = WORKLOADS["prefill"]
    say("prefill workload: generating")
    b = batch_inputs(wl)
    B, T, H, D = len(b["lengths"]), wl.seqlen, wl.H, wl.dk
    d = to_dev(b, torch.bfloat16)
    shp = (B, T, H)
    o, S_T = kda().kda_fwd_chunked(d["q"].view(*shp, D), d["k"].view(*shp, D),
                                   d["v"].view(*shp, D), d["g"].view(*shp, D),
                                   d["beta"].view(*shp))
    torch.cuda.synchronize()
    del d
    assert o.dtype == torch.bfloat16 and o.shape == (B, T, H, D)
    o = o.float().cpu().numpy()
    S_T = S_T.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S_T))
    for n, h in [(0, 0), (1, 17), (2, 31), (3, 5)]:
        check_chain(wl, n, h, T, o[n, :, h], S_T[n, h], "prefill")


def test_long_prefill_sampled_with_carry_over():
    """1 x 65,536 tokens, H = 64, d = 128, bf16, S0 ~ N(0, 0.02): whole run,
    and the same run split in two segments with the first one's S_T handed
    to the second (the split falls inside a chunk)."""
    wl = WORKLOADS["long_prefill"]
    say("long prefill: generating")
    b = batch_inputs(wl)
    T, H, D = wl.seqlen, wl.H, wl.dk
    d = to_dev(b, torch.bfloat16)
    m = kda()
    o, S_T = m.kda_fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["s0"])
    T1 = 40_007
    seg = lambda x, a, c: x[a:c].contiguous()                       # noqa: E731
    names = ("q", "k", "v", "g", "beta")
    o1, S1 = m.kda_fwd_chunked(*(seg(d[x], 0, T1) for x in names), S0=d["s0"])
    o2, S2 = m.kda_fwd_chunked(*(seg(d[x], T1, T) for x in names), S0=S1)
    torch.cuda.synchronize()
    del d
    o = o.float().cpu().numpy()
    S_T = S_T[0].cpu().numpy()
    oc = torch.cat([o1, o2]).float().cpu().numpy()
    S2 = S2[0].cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S_T))
    for h in (0, 37, 63):
        ref = reference(wl, 0, h, T)
        check_chain(wl, 0, h, T, o[:, h], S_T[h], "long", ref)
        check_chain(wl, 0, h, T, oc[:, h], S2[h], "long, two segments", ref)


def test_varlen_sampled():
    """64 sequences, log-uniform lengths in [128, 32768], H = 32, d = 128,
    bf16, decay stress on heads 0..15, beta = 1 on 10 % of the tokens, keys
    repeated inside every tile; packed through cu_seqlens."""
    wl = WORKLOADS["varlen"]
    say("varlen: generating")
    b = batch_inputs(wl)
    lengths, cu = b["lengths"], b["cu_seqlens"]
    d = to_dev(b, torch.bfloat16)
    o, S_T = kda().kda_fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                   cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    del d
    o = o.float().cpu().numpy()
    S_T = S_T.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S_T))
    order = np.argsort(lengths)
    seqs = [int(order[-1]), int(order[0]), int(order[len(order) // 2]), int(order[len(order) // 4])]
    for n in seqs:
        a, c = int(cu[n]), int(cu[n + 1])
        for h in (0, 15, 16, 31):
            check_chain(wl, n, h, c - a, o[a:c, h], S_T[n, h], "varlen")


def test_decode_workload_sampled():
    """256 sequences x 64 heads, d = 128, one step in place, bf16 o."""
    wl = WORKLOADS["decode"]
    say("decode workload: generating")
    b = decode_batch_inputs(wl)
    d = {key: torch.from_numpy(b[key]).cuda().to(torch.bfloat16) for key in ("q", "k", "v")}
    d.update({key: torch.from_numpy(b[key]).cuda() for key in ("g", "beta", "S")})
    o = kda().kda_decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S"])
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    S = d["S"].cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    r = np.random.default_rng(1)
    pick = [(int(n), int(h)) for n, h in zip(r.integers(0, wl.n_seqs, 256),
                                              r.integers(0, wl.H, 256))]
    sel = lambda x: np.stack([x[n, h] for n, h in pick])[:, None]   # noqa: E731
    o_ref, S_ref = ref_decode(sel(b["q"]), sel(b["k"]), sel(b["v"]), sel(b["g"]),
                              sel(b["beta"]), sel(b["S"]))
    eo = err_bf16_out(np.stack([o[n, h] for n, h in pick])[:, None], o_ref)
    es = err(np.stack([S[n, h] for n, h in pick])[:, None], S_ref)
    say(f"  decode 256 sampled heads: o {eo:.2e}  S {es:.2e}")
    assert eo <= TOL and es <= TOL


def test_all_sequences_empty():
    """n_seqs > 0 but every sequence empty: S_T = S0, nothing else written."""
    H, D = 2, 64
    S0 = torch.randn(3, H, D, D, device="cuda")
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    z = lambda *s: torch.zeros(*s, device="cuda")                   # noqa: E731
    o, S_T = kda().kda_fwd_chunked(z(0, H, D).bfloat16(), z(0, H, D).bfloat16(),
                                   z(0, H, D).bfloat16(), z(0, H, D), z(0, H), S0=S0,
                                   cu_seqlens=cu)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(S_T, S0)
