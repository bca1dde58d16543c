"""GPU parity of speculative decoding (kda_decode_verify / _commit / _spec)
through the C ABI against the fp64 oracle (oracle/spec.py).

Tolerance as elsewhere: max |x - ref| / rms(ref) <= 1e-4 (fp32 inputs) or
2e-2 (bf16 inputs; bf16 o with the half-ulp storage allowance)."""
import sys

import numpy as np
import pytest
import torch

from oracle.spec import kda_spec_commit, kda_spec_step, kda_spec_verify
from synth import round_bf16
from tests._gpu_util import err, err_bf16_out

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def kda():
    import gated_delta_rule_95_amd as m
    return m


def drafts(seed, N, K, H, dk, dv, bf16):
    r = np.random.default_rng(seed)
    unit = lambda x: (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)  # noqa
    d = {"q": unit(r.standard_normal((N, K, H, dk))), "k": unit(r.standard_normal((N, K, H, dk))),
         "v": r.standard_normal((N, K, H, dv)).astype(np.float32),
         "g": (-5.0 / (1.0 + np.exp(-r.standard_normal((N, K, H, dk))))).astype(np.float32),
         "beta": (1.0 / (1.0 + np.exp(-r.standard_normal((N, K, H))))).astype(np.float32)}
    if bf16:
        for key in ("q", "k", "v"):
            d[key] = round_bf16(d[key])
    return d


def dev(d, dtype):
    out = {key: torch.from_numpy(d[key]).cuda().to(dtype) for key in ("q", "k", "v")}
    out.update({key: torch.from_numpy(d[key]).cuda() for key in ("g", "beta")})
    return out


SHAPES = [(128, 128), (64, 32), (16, 16), (32, 128), (128, 16)]


@pytest.mark.parametrize("dk,dv", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("K", [1, 4, 16])
def test_verify(dk, dv, dtype, K):
    N, H = 3, 2
    bf = dtype == torch.bfloat16
    d = drafts(dk * 7 + dv + K, N, K, H, dk, dv, bf)
    S = (np.random.default_rng(K).standard_normal((N, H, dk, dv)) * 0.05).astype(np.float32)
    say("verify", dk, dv, dtype, K)
    o_ref = kda_spec_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], S)
    t = dev(d, dtype)
    Sd = torch.from_numpy(S).cuda()
    o = kda().kda_decode_verify(t["q"], t["k"], t["v"], t["g"], t["beta"], Sd)
    torch.cuda.synchronize()
    assert torch.equal(Sd.cpu(), torch.from_numpy(S))          # S is read only
    o = o.float().cpu().numpy()
    e = err_bf16_out(o, o_ref) if bf else err(o, o_ref)
    assert e <= (2e-2 if bf else 1e-4), e


@pytest.mark.parametrize("dk,dv", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_commit(dk, dv, dtype):
    N, H, K = 6, 2, 5
    bf = dtype == torch.bfloat16
    d = drafts(dk + 3 * dv, N, K, H, dk, dv, bf)
    S = (np.random.default_rng(dk).standard_normal((N, H, dk, dv)) * 0.05).astype(np.float32)
    acc = np.array([0, 1, 3, 5, -2, 9], np.int32)               # the last two are clamped
    say("commit", dk, dv, dtype)
    S_ref = kda_spec_commit(d["k"], d["v"], d["g"], d["beta"], acc, S)
    t = dev(d, dtype)
    Sd = torch.from_numpy(S).cuda()
    kda().kda_decode_commit(t["k"], t["v"], t["g"], t["beta"], torch.from_numpy(acc).cuda(), Sd)
    torch.cuda.synchronize()
    Sg = Sd.cpu().numpy()
    assert np.array_equal(Sg[0], S[0]) and np.array_equal(Sg[4], S[4])   # nothing accepted
    assert err(Sg, S_ref) <= (2e-2 if bf else 1e-4)


@pytest.mark.parametrize("dk,dv", [(128, 128), (32, 64)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_spec_step_equals_commit_then_verify(dk, dv, dtype):
    N, H, Kp, K = 4, 3, 4, 3
    bf = dtype == torch.bfloat16
    prev = drafts(11 + dk, N, Kp, H, dk, dv, bf)
    new = drafts(12 + dk, N, K, H, dk, dv, bf)
    S = (np.random.default_rng(5).standard_normal((N, H, dk, dv)) * 0.05).astype(np.float32)
    acc = np.array([2, 0, 4, 1], np.int32)
    say("spec step", dk, dv, dtype)
    o_ref, S_ref = kda_spec_step(prev, acc, new, S)
    m = kda()
    tp, tn = dev(prev, dtype), dev(new, dtype)
    acc_d = torch.from_numpy(acc).cuda()
    Sd = torch.from_numpy(S).cuda()
    o = m.kda_decode_spec(tn["q"], tn["k"], tn["v"], tn["g"], tn["beta"], Sd, prev=tp,
                          n_accept=acc_d)
    # the same through the two separate calls
    S2 = torch.from_numpy(S).cuda()
    m.kda_decode_commit(tp["k"], tp["v"], tp["g"], tp["beta"], acc_d, S2)
    o2 = m.kda_decode_verify(tn["q"], tn["k"], tn["v"], tn["g"], tn["beta"], S2)
    torch.cuda.synchronize()
    assert torch.equal(Sd, S2) and torch.equal(o, o2)
    o = o.float().cpu().numpy()
    tol = 2e-2 if bf else 1e-4
    assert (err_bf16_out(o, o_ref) if bf else err(o, o_ref)) <= tol
    assert err(Sd.cpu().numpy(), S_ref) <= tol


def test_verify_single_draft_matches_decode_step():
    N, H, D = 5, 4, 128
    d = drafts(99, N, 1, H, D, D, True)
    S = (np.random.default_rng(9).standard_normal((N, H, D, D)) * 0.05).astype(np.float32)
    m = kda()
    t = dev(d, torch.bfloat16)
    Sd = torch.from_numpy(S).cuda()
    o1 = m.kda_decode_verify(t["q"], t["k"], t["v"], t["g"], t["beta"], Sd,
                             out_dtype=torch.float32)
    o2 = m.kda_decode_step(t["q"][:, 0].contiguous(), t["k"][:, 0].contiguous(),
                           t["v"][:, 0].contiguous(), t["g"][:, 0].contiguous(),
                           t["beta"][:, 0].contiguous(), Sd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert err(o1[:, 0].cpu().numpy(), o2.cpu().numpy().astype(np.float64)) <= 1e-5


@pytest.mark.timeout(600)
def test_spec_decode_workload_all_heads():
    """The decode workload's shape (256 sequences x 64 heads, d = 128, bf16)
    with 4 previous drafts (accepted counts 0..4) and 4 new drafts; every
    head's o and committed state against the oracle."""
    N, H, D, Kp, K = 256, 64, 128, 4, 4
    prev = drafts(1234, N, Kp, H, D, D, True)
    new = drafts(1235, N, K, H, D, D, True)
    S = (np.random.default_rng(77).standard_normal((N, H, D, D)) * 0.05).astype(np.float32)
    acc = np.random.default_rng(78).integers(0, Kp + 1, N).astype(np.int32)
    say("spec step, decode workload shape")
    tp, tn = dev(prev, torch.bfloat16), dev(new, torch.bfloat16)
    Sd = torch.from_numpy(S).cuda()
    o = kda().kda_decode_spec(tn["q"], tn["k"], tn["v"], tn["g"], tn["beta"], Sd, prev=tp,
                              n_accept=torch.from_numpy(acc).cuda())
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    Sg = Sd.cpu().numpy()
    worst_o, worst_s, sq_o, sq_s = 0.0, 0.0, 0.0, 0.0
    from tests._gpu_util import half_ulp_bf16
    for n0 in range(0, N, 32):
        sl = slice(n0, n0 + 32)
        o_ref, S_ref = kda_spec_step({key: x[sl] for key, x in prev.items()}, acc[sl],
                                     {key: x[sl] for key, x in new.items()}, S[sl])
        dev_o = np.maximum(np.abs(o[sl] - o_ref) - half_ulp_bf16(o_ref), 0.0)
        worst_o = max(worst_o, float(dev_o.max()))
        worst_s = max(worst_s, float(np.abs(Sg[sl] - S_ref).max()))
        sq_o += float(np.sum(o_ref ** 2))
        sq_s += float(np.sum(S_ref ** 2))
    eo = worst_o / np.sqrt(sq_o / o.size)
    es = worst_s / np.sqrt(sq_s / Sg.size)
    say(f"  all {N} x {H} heads: o {eo:.2e}  S {es:.2e}")
    assert eo <= 2e-2 and es <= 2e-2
