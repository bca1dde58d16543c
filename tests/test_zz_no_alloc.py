"""GPU test of kda_fwd_chunked_noalloc (the prefill for callers that cannot
allocate): called through the C ABI, its output must match
kda_fwd_chunked's with a caller workspace, on two calls in a row, the
second smaller, both on the sequence-split path that uses the scratch."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from oracle import clib
from tests._gpu_util import err, err_bf16_out, random_batch, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def call_noalloc(lib, d, ns, T, H, D, S0, o, S_T):
    p = lambda t: None if t is None else t.data_ptr()          # noqa: E731
    stream = torch.cuda.current_stream().cuda_stream
    return lib.kda_fwd_chunked_noalloc(p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]),
                                       p(d["beta"]), p(S0), None, ns, ns * T, H, D, D, 1, 1,
                                       p(o), p(S_T), stream)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_entry_point(order):
    import gated_delta_rule_95_amd as kda
    from gated_delta_rule_95_amd import _lib
    lib = _lib.load()
    D = 128
    for (ns, T, H, seed) in [(1, 4096, 4, 31), (1, 3001, 2, 32)]:
        need = kda.kda_fwd_workspace_bytes(ns, ns * T, H, D, D, torch.bfloat16)
        say(f"noalloc: n_seqs {ns} T {T} H {H}: scratch {need} bytes")
        assert 0 < need <= 64 << 20
        b = random_batch(seed, [T] * ns, H=H, dk=D, dv=D)
        d = to_dev(b, torch.bfloat16)
        o_na = torch.full((ns * T, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        S_na = torch.full((ns, H, D, D), float("nan"), device="cuda")
        st = call_noalloc(lib, d, ns, T, H, D, d["s0"], o_na, S_na)
        assert st == 0, _lib.last_error()
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        o_ws, S_ws = kda.kda_fwd_chunked(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["s0"],
                                         workspace=ws)
        torch.cuda.synchronize()
        o_na, S_na = o_na.float().cpu().numpy(), S_na.cpu().numpy()
        o_ws, S_ws = o_ws.float().cpu().numpy(), S_ws.cpu().numpy()
        o_ref, S_ref, _ = clib.fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], b["cu_seqlens"],
                                   b["s0"])
        e1, e2 = err(o_na, o_ws.astype(np.float64)), err(S_na, S_ws.astype(np.float64))
        e3, e4 = err_bf16_out(o_na, o_ref), err(S_na, S_ref)
        say(f"  vs workspace entry point: o {e1:.2e} S_T {e2:.2e} "
            f"(bit-identical: {np.array_equal(o_na, o_ws) and np.array_equal(S_na, S_ws)}); "
            f"vs oracle: o {e3:.2e} S_T {e4:.2e}")
        assert e1 <= 2e-2 and e2 <= 2e-2 and e3 <= 2e-2 and e4 <= 2e-2
