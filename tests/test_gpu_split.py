"""GPU parity of the sequence-split prefill path (segments side by side,
affine summaries, scan over segments, correction), through the C ABI.

Shapes are chosen with few (sequence, head) chains and long sequences, where
kda_fwd_workspace_bytes is nonzero, i.e. the library does split; every test
asserts that first.  Results are compared with the fp64 oracle at the usual
tolerance (2e-2 bf16, 1e-4 fp32, max |x - ref| / rms(ref)) and with the
single-pass path.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import clib
from tests._gpu_util import err, err_bf16_out, random_batch, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def kda():
    import gated_delta_rule_95_amd as m
    return m


def equal_batch(seed, n_seqs, T, H, dk, dv, s0, bf16):
    b = random_batch(seed, [T] * n_seqs, H=H, dk=dk, dv=dv, s0=s0, bf16=bf16)
    return b


def run(b, n_seqs, T, dtype, out_dtype, workspace, with_s0=True, final=True):
    d = to_dev(b, dtype)
    H, dk = d["q"].shape[1], d["q"].shape[2]
    dv = d["v"].shape[2]
    shp = (n_seqs, T, H)
    o, ST = kda().kda_fwd_chunked(d["q"].view(*shp, dk), d["k"].view(*shp, dk),
                                  d["v"].view(*shp, dv), d["g"].view(*shp, dk),
                                  d["beta"].view(*shp), S0=d.get("s0") if with_s0 else None,
                                  out_dtype=out_dtype, output_final_state=final,
                                  workspace=workspace)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().reshape(n_seqs * T, H, dv)
    return o, (ST.cpu().numpy() if ST is not None else None)


CASES = [
    # n_seqs, T, H, dk, dv, dtype, out_dtype, S0, S_T
    (1, 4096, 4, 128, 128, torch.bfloat16, torch.bfloat16, True, True),
    (1, 3001, 2, 128, 128, torch.bfloat16, torch.float32, False, True),
    (2, 2048, 1, 128, 128, torch.bfloat16, torch.bfloat16, True, False),
    (1, 6000, 3, 64, 64, torch.float32, torch.float32, True, True),
    (1, 2500, 2, 32, 128, torch.bfloat16, torch.float32, True, True),
    (1, 2048, 2, 128, 32, torch.float32, torch.float32, False, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "n%d_T%d_H%d_dk%d_dv%d_%s" % (
    c[0], c[1], c[2], c[3], c[4], "bf16" if c[5] == torch.bfloat16 else "f32"))
def test_split_matches_oracle_and_single_pass(case):
    ns, T, H, dk, dv, dt, odt, s0, final = case
    need = kda().kda_fwd_workspace_bytes(ns, ns * T, H, dk, dv, dt)
    say("split case", case, "workspace bytes", need)
    assert need > 0, "these sizes are meant to take the sequence-split path"
    b = equal_batch(100 + T + H, ns, T, H, dk, dv, s0, dt == torch.bfloat16)
    o_ref, S_ref, _ = clib.fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], b["cu_seqlens"],
                               b.get("s0") if s0 else None)
    o_s, S_s = run(b, ns, T, dt, odt, True, with_s0=s0, final=final)
    o_1, S_1 = run(b, ns, T, dt, odt, False, with_s0=s0, final=final)
    tol = 2e-2 if dt == torch.bfloat16 else 1e-4
    metric = err_bf16_out if odt == torch.bfloat16 else err
    eo_s, eo_1 = metric(o_s, o_ref), metric(o_1, o_ref)
    say(f"  o: split {eo_s:.2e} single {eo_1:.2e}")
    assert eo_s <= tol and eo_1 <= tol
    if final:
        es_s, es_1 = err(S_s, S_ref), err(S_1, S_ref)
        say(f"  S_T: split {es_s:.2e} single {es_1:.2e}")
        assert es_s <= tol and es_1 <= tol
    else:
        assert S_s is None and S_1 is None


def test_split_caller_workspace_reused_and_deterministic():
    """A caller-owned uint8 workspace of exactly the queried size, used by two
    calls in a row: both give the same, correct result."""
    ns, T, H, d = 1, 4096, 4, 128
    need = kda().kda_fwd_workspace_bytes(ns, T, H, d, d, torch.bfloat16)
    assert need > 0
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")
    b = equal_batch(7, ns, T, H, d, d, True, True)
    o1, S1 = run(b, ns, T, torch.bfloat16, torch.bfloat16, ws)
    o2, S2 = run(b, ns, T, torch.bfloat16, torch.bfloat16, ws)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    o_ref, S_ref, _ = clib.fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], b["cu_seqlens"],
                               b["s0"])
    assert err_bf16_out(o1, o_ref) <= 2e-2 and err(S1, S_ref) <= 2e-2


def test_split_rejects_small_workspace():
    ns, T, H, d = 1, 4096, 4, 128
    need = kda().kda_fwd_workspace_bytes(ns, T, H, d, d, torch.bfloat16)
    assert need > 0
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    b = equal_batch(8, ns, T, H, d, d, True, True)
    with pytest.raises(kda().KDAError) as ei:
        run(b, ns, T, torch.bfloat16, torch.bfloat16, ws)
    assert ei.value.status == 1
    assert "below" in str(ei.value)
