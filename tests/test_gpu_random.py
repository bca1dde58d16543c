"""Seeded random configurations of every entry point against the fp64 oracle
(GPU, through the C ABI): key and value widths, head counts, packed ragged
or equal-length batches (empty and one-token sequences included), input
and output dtypes, S0 given or not, S_T kept or not.  The structured tests
pin the named shapes; these cover their combinations.

Bars as elsewhere: max |x - ref| / rms(ref) <= 1e-4 (fp32 inputs) or 2e-2
(bf16 inputs; a bf16-stored o with the half-ulp storage allowance), except
dg from fp32 inputs, 2e-4: the chunked algebra forms it as the difference of
the chunk's total-decay term and the per-token log terms, each up to ~30x
larger than dg and rounded to fp32, so its worst elements carry ~3e-6
relative error, and a heavy-tailed dg (max/rms ~50) lifts max|err|/rms to
about 1.2e-4."""
import sys

import numpy as np
import pytest
import torch

from oracle import clib
from oracle.prologue import kda_prologue
from oracle.recurrence import kda_decode_step as ref_decode
from synth import round_bf16
from tests._gpu_util import err, err_bf16_out

pytestmark = pytest.mark.gpu
WIDTHS = (16, 32, 64, 128)
N_CASES = 24


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def kda():
    import gated_delta_rule_95_amd as m
    return m


def tol(bf16):
    return 2e-2 if bf16 else 1e-4


def draw(seed):
    """One configuration: widths, heads, lengths, dtype and options."""
    r = np.random.default_rng(seed)
    dk, dv = (int(x) for x in r.choice(WIDTHS, 2))
    H = int(r.integers(1, 5))
    ns = int(r.integers(1, 6))
    equal = bool(r.random() < 0.25)
    if equal:
        lengths = np.full(ns, int(r.integers(1, 320)))
    else:
        lengths = r.integers(0, 400, ns)
        special = r.random(ns)
        lengths[special < 0.15] = 0
        lengths[(special >= 0.15) & (special < 0.3)] = 1
        lengths[(special >= 0.3) & (special < 0.4)] = 16 * r.integers(1, 6)
    return {"dk": dk, "dv": dv, "H": H, "lengths": lengths.astype(np.int64), "equal": equal,
            "bf16": bool(r.random() < 0.6), "s0": bool(r.random() < 0.6),
            "final": bool(r.random() < 0.8), "out_f32": bool(r.random() < 0.3), "rng": r}


def inputs(c):
    r, H, dk, dv = c["rng"], c["H"], c["dk"], c["dv"]
    cu = np.concatenate([[0], np.cumsum(c["lengths"])]).astype(np.int32)
    N = int(cu[-1])

    def unit(x):
        return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)
    d = {"q": unit(r.standard_normal((N, H, dk))), "k": unit(r.standard_normal((N, H, dk))),
         "v": r.standard_normal((N, H, dv)).astype(np.float32),
         "g": (-5.0 / (1.0 + np.exp(-1.5 * r.standard_normal((N, H, dk))))).astype(np.float32),
         "beta": (1.0 / (1.0 + np.exp(-r.standard_normal((N, H))))).astype(np.float32),
         "cu_seqlens": cu}
    if c["bf16"]:
        for key in ("q", "k", "v"):
            d[key] = round_bf16(d[key])
    if c["s0"]:
        d["s0"] = (0.5 * r.standard_normal((len(cu) - 1, H, dk, dv))).astype(np.float32)
    return d


def lead_view(c, x):
    """[N, ...] -> [B, T, ...] for an equal-length batch without cu_seqlens."""
    if not c["equal"]:
        return x
    B, T = len(c["lengths"]), int(c["lengths"][0])
    return x.view((B, T) + tuple(x.shape[1:]))


def check_o(c, o, o_ref, tag):
    if o_ref.size == 0:
        assert o.size == 0
        return
    if c["bf16"] and not c["out_f32"]:
        e = err_bf16_out(o, o_ref)
    else:
        e = err(o, o_ref)
    say(f"  {tag} o {e:.2e}")
    assert e <= tol(c["bf16"]), (tag, e)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_prefill(case):
    c = draw(7000 + case)
    d = inputs(c)
    say("prefill", case, {key: c[key] for key in ("dk", "dv", "H", "equal", "bf16", "s0",
                                                  "final", "out_f32")}, c["lengths"].tolist())
    o_ref, S_ref, _ = clib.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                               d.get("s0"))
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    t = {key: lead_view(c, torch.from_numpy(d[key]).cuda().to(dt)) for key in ("q", "k", "v")}
    g = lead_view(c, torch.from_numpy(d["g"]).cuda())
    beta = lead_view(c, torch.from_numpy(d["beta"]).cuda())
    cu = None if c["equal"] else torch.from_numpy(d["cu_seqlens"]).cuda()
    S0 = torch.from_numpy(d["s0"]).cuda() if c["s0"] else None
    o, S = kda().kda_fwd_chunked(t["q"], t["k"], t["v"], g, beta, S0=S0, cu_seqlens=cu,
                                 out_dtype=torch.float32 if c["out_f32"] else None,
                                 output_final_state=c["final"])
    torch.cuda.synchronize()
    N = int(d["cu_seqlens"][-1])
    check_o(c, o.float().cpu().numpy().reshape(N, c["H"], c["dv"]), o_ref, "prefill")
    if c["final"]:
        e = err(S.cpu().numpy(), S_ref)
        say(f"  prefill S_T {e:.2e}")
        assert e <= tol(c["bf16"])
    else:
        assert S is None


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_gated(case):
    c = draw(8000 + case)
    r, H, dk, dv = c["rng"], c["H"], c["dk"], c["dv"]
    cu = np.concatenate([[0], np.cumsum(c["lengths"])]).astype(np.int32)
    N = int(cu[-1])
    scale = np.exp(r.uniform(np.log(0.05), np.log(20.0), (N, H, 1))).astype(np.float32)
    d = {"q": r.standard_normal((N, H, dk)).astype(np.float32) * scale,
         "k": r.standard_normal((N, H, dk)).astype(np.float32) * scale[:, ::-1],
         "v": r.standard_normal((N, H, dv)).astype(np.float32),
         "z": (1.5 * r.standard_normal((N, H, dk))).astype(np.float32),
         "b": r.standard_normal((N, H)).astype(np.float32),
         "A_log": (0.5 * r.standard_normal(H)).astype(np.float32)}
    if c["bf16"]:
        for key in ("q", "k", "v", "z", "b"):
            d[key] = round_bf16(d[key])
    s0 = (0.3 * r.standard_normal((len(cu) - 1, H, dk, dv))).astype(np.float32) \
        if c["s0"] else None
    say("gated", case, {key: c[key] for key in ("dk", "dv", "H", "equal", "bf16", "s0")},
        c["lengths"].tolist())
    qn, kn, g, beta = kda_prologue(d["q"], d["k"], d["z"], d["A_log"], d["b"])
    f = lambda x: np.asarray(x, np.float32)                   # noqa: E731
    o_ref, S_ref, _ = clib.fwd(f(qn), f(kn), d["v"], f(g), f(beta), cu, s0)
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    t = {key: lead_view(c, torch.from_numpy(d[key]).cuda().to(dt))
         for key in ("q", "k", "v", "z", "b")}
    o, S = kda().kda_fwd_chunked_gated(
        t["q"], t["k"], t["v"], t["z"], torch.from_numpy(d["A_log"]).cuda(), t["b"],
        S0=None if s0 is None else torch.from_numpy(s0).cuda(),
        cu_seqlens=None if c["equal"] else torch.from_numpy(cu).cuda(),
        out_dtype=torch.float32 if c["out_f32"] else None)
    torch.cuda.synchronize()
    check_o(c, o.float().cpu().numpy().reshape(N, H, dv), o_ref, "gated")
    e = err(S.cpu().numpy(), S_ref)
    say(f"  gated S_T {e:.2e}")
    assert e <= tol(c["bf16"])


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_backward(case):
    c = draw(9000 + case)
    d = inputs(c)
    r, H, dk, dv = c["rng"], c["H"], c["dk"], c["dv"]
    N, ns = int(d["cu_seqlens"][-1]), len(d["cu_seqlens"]) - 1
    dO = r.standard_normal((N, H, dv)).astype(np.float32)
    if c["bf16"]:
        dO = round_bf16(dO)
    dST = r.standard_normal((ns, H, dk, dv)).astype(np.float32) if c["final"] else None
    say("backward", case, {key: c[key] for key in ("dk", "dv", "H", "equal", "bf16", "s0",
                                                   "final")}, c["lengths"].tolist())
    ref = clib.vjp(d["q"], d["k"], d["v"], d["g"], d["beta"], dO, d["cu_seqlens"],
                   d.get("s0"), dST)[:6]
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    t = {key: lead_view(c, torch.from_numpy(d[key]).cuda().to(dt)) for key in ("q", "k", "v")}
    got = kda().kda_bwd_chunked(
        t["q"], t["k"], t["v"], lead_view(c, torch.from_numpy(d["g"]).cuda()),
        lead_view(c, torch.from_numpy(d["beta"]).cuda()),
        lead_view(c, torch.from_numpy(dO).cuda().to(dt)),
        S0=torch.from_numpy(d["s0"]).cuda() if c["s0"] else None,
        dS_T=None if dST is None else torch.from_numpy(dST).cuda(),
        cu_seqlens=None if c["equal"] else torch.from_numpy(d["cu_seqlens"]).cuda())
    torch.cuda.synchronize()
    shapes = ((N, H, dk), (N, H, dk), (N, H, dv), (N, H, dk), (N, H), (ns, H, dk, dv))
    for name, x, y, shp in zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), got, ref, shapes):
        x = x.float().cpu().numpy().reshape(shp)
        e = err(x, y) if np.all(np.isfinite(x)) else float("inf")
        say(f"  backward {name} {e:.2e}")
        bar = 2e-4 if (name == "dg" and not c["bf16"]) else tol(c["bf16"])
        assert e <= bar, (name, e)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_decode(case):
    c = draw(10000 + case)
    r, H, dk, dv = c["rng"], c["H"], c["dk"], c["dv"]
    N = int(r.integers(1, 40))
    c["lengths"] = np.ones(N, np.int64)
    c["equal"] = False
    d = inputs(c)
    S = (0.05 * r.standard_normal((N, H, dk, dv))).astype(np.float32)
    say("decode", case, {key: c[key] for key in ("dk", "dv", "H", "bf16", "out_f32")}, N)
    o_ref, S_ref = ref_decode(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    t = {key: torch.from_numpy(d[key]).cuda().to(dt) for key in ("q", "k", "v")}
    Sd = torch.from_numpy(S).cuda()
    o = kda().kda_decode_step(t["q"], t["k"], t["v"], torch.from_numpy(d["g"]).cuda(),
                              torch.from_numpy(d["beta"]).cuda(), Sd,
                              out_dtype=torch.float32 if c["out_f32"] else None)
    torch.cuda.synchronize()
    check_o(c, o.float().cpu().numpy(), o_ref, "decode")
    e = err(Sd.cpu().numpy(), S_ref)
    say(f"  decode S {e:.2e}")
    assert e <= tol(c["bf16"])
