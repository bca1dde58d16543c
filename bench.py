#!/usr/bin/env python3
"""KDA benchmark on one MI355X: chunked prefill tokens/s + decode state GB/s.

A step is one pass over the whole hot path on synthetic inputs already
resident in HBM:
  * kda_fwd_chunked on the prefill workload (default: 4 sequences x 4096
    tokens, H = 32, d_k = d_v = 128, bf16 q/k/v and o, fp32 g/beta, S0 = 0,
    S_T written), and
  * kda_decode_step on the decode workload (256 sequences x 64 heads,
    d = 128, fp32 state updated in place).
Each launch is bracketed by HIP events recorded on the stream it runs on.
`value` is prefill tokens per second over the K timed launches; the decode
state bandwidth and both roofline fractions ride along in the same line.

    python bench.py [--steps K] [--warmup W] [--workload prefill|long_prefill|varlen]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
SPEC_K = 4                       # drafts per speculative step (previous and new)
SEED_ACCEPT = 0x4B4441 + 17      # seeded acceptance counts of the speculative leg
SEED_COTANGENT = 0x4B4441 + 23   # seeded cotangents of the backward leg
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 matrix, published
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_bytes(tokens: int, H: int, dk: int, dv: int, n_seqs: int, s0: bool) -> int:
    """Algorithmic HBM bytes of one prefill launch: q, k (bf16, d_k), v (bf16,
    d_v), g (fp32, d_k), beta (fp32), o (bf16, d_v) per token-head, plus the
    fp32 S_T write (and S0 read) per (sequence, head)."""
    per_th = 2 * dk * 2 + 2 * dv + 4 * dk + 4 + 2 * dv
    state = n_seqs * H * dk * dv * 4
    return tokens * H * per_th + state * (2 if s0 else 1)


def prefill_flops(tokens: int, H: int, dk: int, dv: int) -> int:
    """Algorithmic flops at the 16-token tile: 6 d_k d_v + 16 (3 d_k + 2 d_v)
    per token-head (state products + intra-tile products)."""
    return tokens * H * (6 * dk * dv + 16 * (3 * dk + 2 * dv))


def gated_prefill_bytes(tokens: int, H: int, dk: int, dv: int, n_seqs: int) -> int:
    """Algorithmic bytes of the fused-prologue prefill: q, k, z (bf16, d_k),
    v and o (bf16, d_v), b (bf16) per token-head, A_log, the S_T write."""
    return tokens * H * (3 * 2 * dk + 2 * 2 * dv + 2) + 4 * H + n_seqs * H * dk * dv * 4


def decode_bytes(N: int, H: int, dk: int, dv: int) -> tuple:
    state = N * H * dk * dv * 4 * 2                    # read + write
    other = N * H * (2 * dk * 2 + 2 * dv + 4 * dk + 4 + 2 * dv)
    return state, state + other


def spec_bytes(N: int, H: int, dk: int, dv: int, K: int, K_prev: int) -> tuple:
    """One fused speculative step: the state read and written once; per
    previous draft k, v (bf16), g, beta; per new draft q, k, v (bf16), g,
    beta and o (bf16); the accepted counts."""
    state = N * H * dk * dv * 4 * 2
    prev = N * K_prev * H * (2 * dk + 2 * dv + 4 * dk + 4)
    new = N * K * H * (2 * dk * 2 + 2 * dv + 4 * dk + 4 + 2 * dv)
    return state, state + prev + new + 4 * N


def backward_bytes(tokens: int, H: int, dk: int, dv: int, n_seqs: int, s0: bool) -> int:
    """Algorithmic HBM bytes of one kda_bwd_chunked call: read q, k, v, dO
    (bf16), g (fp32 [N,H,dk]), beta, S0 and dS_T once; write dq, dk, dg (fp32
    [N,H,dk]), dv (fp32 [N,H,dv]), dbeta and dS0 once.  Checkpointed chunk
    states and per-chunk partials are the implementation's own traffic."""
    per_tok = H * ((2 * dk + 2 * dv) * 2 + dk * 4 + 4 + 3 * dk * 4 + dv * 4 + 4)
    st = n_seqs * H * dk * dv * 4
    return tokens * per_tok + st * (3 if s0 else 2)


def counter_record(workload: str, kernel: str):
    """The committed rocprofv3 counter summary of `kernel` (a class name of
    profile_summary.kernel_class) on `workload`, or None: only a record
    taken on this kernel's current sources and on this very workload counts."""
    from profile_summary import source_hash
    try:
        with open(os.path.join(PROFILE_DIR, f"pmc_{workload}.json")) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if rec.get("workload") != workload or not k or \
            k.get("source_sha256_16") != source_hash(kernel):
        return None
    return k


def attach_counters(roofline: dict, workload: str, kernel: str) -> dict:
    """traffic = HBM bytes per dispatch from the counter record (null without
    one); the matrix-core and vector-ALU busy fractions ride along."""
    k = counter_record(workload, kernel)
    roofline["traffic"] = None if k is None else k.get("hbm_bytes_per_dispatch")
    if k is not None and "mfma_busy_pct" in k:
        roofline["counters"] = {key: k[key] for key in
                                ("mfma_busy_pct", "valu_busy_pct", "lds_bank_conflict_pct",
                                 "mfma_bf16_flops") if key in k}
    return roofline


def attach_counters_sum(roofline: dict, workload: str, kernels) -> dict:
    """traffic of a call made of several kernels: the sum of their HBM bytes
    per dispatch, when every one of them has a current counter record (null
    otherwise), and each kernel's own figure beside it."""
    recs = [counter_record(workload, k) for k in kernels]
    ok = all(r is not None and "hbm_bytes_per_dispatch" in r for r in recs)
    roofline["traffic"] = sum(r["hbm_bytes_per_dispatch"] for r in recs) if ok else None
    if ok:
        roofline["traffic_by_kernel"] = {k: r["hbm_bytes_per_dispatch"]
                                         for k, r in zip(kernels, recs)}
    return roofline


def host_cpu() -> dict:
    """What the host offers the oracle: logical CPUs, the CPUs this process
    may run on, and the CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"nproc": os.cpu_count() or 1, "usable": usable, "model": model}


def cpu_baseline(threads: int):
    """The fp64 C oracle on the whole prefill workload (4 sequences x 4096
    tokens x 32 heads, d = 128; about 20 core-seconds) on `threads` host
    threads, and on one thread over 4 of its 128 (sequence, head) chains."""
    from oracle import clib
    from synth import WORKLOADS, batch_inputs
    wl = WORKLOADS["prefill"]
    b = batch_inputs(wl)
    tokens = int(b["cu_seqlens"][-1])
    t0 = time.perf_counter()
    _, _, used = clib.fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], b["cu_seqlens"], None,
                          want_o=True, threads=threads)
    dt = time.perf_counter() - t0
    # one thread, heads 0..3 of sequence 0 (4 chains of 4096 tokens): tokens/s
    # scaled to all 32 heads, the unit of the whole-workload figure
    one = {key: b[key][:wl.seqlen, :4] for key in ("q", "k", "v", "g", "beta")}
    t1 = time.perf_counter()
    clib.fwd(one["q"], one["k"], one["v"], one["g"], one["beta"],
             [0, wl.seqlen], None, want_o=True, threads=1)
    dt1 = time.perf_counter() - t1
    one_core = wl.seqlen * 4 / wl.H / dt1
    host = host_cpu()
    # fp64 work at the recurrence's 7 d^2 flops per token-head
    flops = 7.0 * wl.dk * wl.dv * tokens * wl.H
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "one_core_value": one_core, "fp64_gflops": flops / dt / 1e9,
            "one_core_fp64_gflops": 7.0 * wl.dk * wl.dv * wl.seqlen * 4 / dt1 / 1e9,
            "host": host,
            "sample": f"fp64 C oracle (token-by-token, OpenMP over (sequence, head)) on the "
                      f"whole prefill workload: {len(b['lengths'])} seqs x {wl.seqlen} tokens x "
                      f"{wl.H} heads, d=128; {dt:.2f} s wall on {used} threads "
                      f"({host['usable']} usable of {host['nproc']} logical CPUs, "
                      f"{host['model']}); one thread: 4 chains of 4096 tokens in {dt1:.2f} s, "
                      f"scaled to 32 heads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first ~100 launches run at lower clocks; the default warmup reaches
    # the steady state before the timed region
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "long_prefill", "varlen", "varlen_1m"])
    ap.add_argument("--heads", type=int, default=0,
                    help="override the workload's head count (split-threshold study)")
    ap.add_argument("--no-split", action="store_true",
                    help="prefill without a workspace: the single-pass kernel only")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-gated", action="store_true",
                    help="skip the fused-prologue prefill leg")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the chunked-backward leg")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this KDA build runs on exactly one GPU (no sharding, no "
              "collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from gated_delta_rule_95_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    import gated_delta_rule_95_amd as kda
    from synth import WORKLOADS, batch_inputs, decode_batch_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---------------- inputs (generated on the host, seeded) ----------------
    wl = WORKLOADS[args.workload]
    if args.heads:
        import dataclasses
        wl = dataclasses.replace(wl, H=args.heads)
    t0 = time.perf_counter()
    b = batch_inputs(wl)
    log(f"[bench] generated {args.workload}: {int(b['cu_seqlens'][-1])} tokens, "
        f"{len(b['lengths'])} seqs in {time.perf_counter() - t0:.1f}s")
    dt_in = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    P = {key: torch.from_numpy(b[key]).to(dev).to(dt_in) for key in ("q", "k", "v")}
    P.update({key: torch.from_numpy(b[key]).to(dev) for key in ("g", "beta")})
    S0 = torch.from_numpy(b["s0"]).to(dev) if "s0" in b else None
    n_seqs = len(b["lengths"])
    tokens = int(b["cu_seqlens"][-1])
    scan_depth = -(-int(max(b["lengths"])) // 16)     # sequential chunks of the longest chain
    equal = wl.seqlen is not None
    cu = None if equal else torch.from_numpy(b["cu_seqlens"]).to(dev)
    if equal:
        shp = (n_seqs, wl.seqlen, wl.H)
        P = {key: (t.view(*shp, -1) if t.dim() == 3 else t.view(*shp)) for key, t in P.items()}
    o = torch.empty(P["v"].shape, dtype=dt_in, device=dev)
    S_T = torch.empty((n_seqs, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=dev)
    del b
    # the workspace of the sequence-split path is allocated once, outside the
    # timed region (the library itself allocates nothing)
    ws_bytes = 0 if (args.no_split or not equal) else \
        kda.kda_fwd_workspace_bytes(n_seqs, tokens, wl.H, wl.dk, wl.dv, dt_in)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else False

    def run_prefill():
        kda.kda_fwd_chunked(P["q"], P["k"], P["v"], P["g"], P["beta"], S0=S0, cu_seqlens=cu,
                            o=o, S_T=S_T, workspace=ws)

    # the same prefill with the gate and q/k preprocessing fused in, from
    # the workload's raw pre-activation draws (A_log = 0); default workload only
    gated = None
    if args.workload == "prefill" and not args.no_gated:
        rb = batch_inputs(wl, raw=True)
        gated = {key: torch.from_numpy(rb[key]).to(dev).to(dt_in) for key in ("q", "k", "v", "z")}
        gated["b"] = torch.from_numpy(rb["b"]).to(dev).to(dt_in)
        shp = (n_seqs, wl.seqlen, wl.H)
        gated = {key: (t.view(*shp, -1) if t.dim() == 3 else t.view(*shp))
                 for key, t in gated.items()}
        gated["A_log"] = torch.zeros(wl.H, device=dev)
        del rb

    def run_gated():
        gp = gated
        kda.kda_fwd_chunked_gated(gp["q"], gp["k"], gp["v"], gp["z"], gp["A_log"], gp["b"],
                                  o=o, S_T=S_T, workspace=ws)

    # the chunked backward of the same prefill, with seeded random cotangents
    # dO (o's shape and dtype) and dS_T; its workspace allocated once here
    bwd = None
    if args.workload == "prefill" and not args.no_backward:
        r = np.random.default_rng(SEED_COTANGENT)
        bwd = {"dO": torch.from_numpy(r.standard_normal(tuple(o.shape), np.float32)).to(dev)
               .to(dt_in),
               "dS_T": torch.from_numpy(r.standard_normal(tuple(S_T.shape), np.float32)).to(dev)}
        bwd["ws"] = torch.empty(kda.kda_bwd_workspace_bytes(n_seqs, tokens, wl.H, wl.dk,
                                                            wl.dv), dtype=torch.uint8, device=dev)

    def run_backward():
        kda.kda_bwd_chunked(P["q"], P["k"], P["v"], P["g"], P["beta"], bwd["dO"], S0=S0,
                            dS_T=bwd["dS_T"], cu_seqlens=cu, workspace=bwd["ws"])

    dec = None
    if not args.no_decode:
        dw = WORKLOADS["decode"]
        d = decode_batch_inputs(dw)
        dec = {key: torch.from_numpy(d[key]).to(dev).to(torch.bfloat16) for key in ("q", "k", "v")}
        dec.update({key: torch.from_numpy(d[key]).to(dev) for key in ("g", "beta", "S")})
        dec["o"] = torch.empty((dw.n_seqs, dw.H, dw.dv), dtype=torch.bfloat16, device=dev)
        del d

    def run_decode():
        kda.kda_decode_step(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], dec["S"],
                            o=dec["o"])

    # speculative step at the decode workload's shape: the previous step's
    # SPEC_K drafts (a seeded number of them accepted per sequence) are
    # committed and SPEC_K new drafts verified, in one pass over the state
    spec = None
    if dec:
        from synth import draft_batch_inputs
        dw = WORKLOADS["decode"]
        nd, pd = draft_batch_inputs(dw, SPEC_K, 1), draft_batch_inputs(dw, SPEC_K, 2)
        tod = lambda x, key: (torch.from_numpy(x[key]).to(dev).to(torch.bfloat16)   # noqa
                              if key in ("q", "k", "v") else torch.from_numpy(x[key]).to(dev))
        spec = {"new": {key: tod(nd, key) for key in nd}, "prev": {key: tod(pd, key) for key in pd},
                "acc": torch.from_numpy(np.random.default_rng(SEED_ACCEPT).integers(
                    0, SPEC_K + 1, dw.n_seqs).astype(np.int32)).to(dev),
                "S": dec["S"].clone(),
                "o": torch.empty((dw.n_seqs, SPEC_K, dw.H, dw.dv), dtype=torch.bfloat16,
                                 device=dev)}
        del nd, pd

    def run_spec():
        n = spec["new"]
        kda.kda_decode_spec(n["q"], n["k"], n["v"], n["g"], n["beta"], spec["S"],
                            prev=spec["prev"], n_accept=spec["acc"], o=spec["o"])

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        log(f"[bench] calibration copy: {args.calib_copy_mib} MiB read + written")
        del src, dst

    # ---------------- warmup ----------------
    for _ in range(args.warmup):
        run_prefill()
        if gated:
            run_gated()
        if bwd:
            run_backward()
        if dec:
            run_decode()
            run_spec()
    torch.cuda.synchronize(dev)
    log(f"[bench] warmup {args.warmup} done")

    # ---------------- timed steps ----------------
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(10)] for _ in range(K)]
    torch.cuda.synchronize(dev)
    wall0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        run_prefill()
        ev[i][1].record(stream)
        if gated:
            ev[i][6].record(stream)
            run_gated()
            ev[i][7].record(stream)
        if bwd:
            ev[i][8].record(stream)
            run_backward()
            ev[i][9].record(stream)
        if dec:
            ev[i][2].record(stream)
            run_decode()
            ev[i][3].record(stream)
            ev[i][4].record(stream)
            run_spec()
            ev[i][5].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall0
    pf_ms = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)])
    dc_ms = np.array([ev[i][2].elapsed_time(ev[i][3]) for i in range(K)]) if dec else None
    sp_ms = np.array([ev[i][4].elapsed_time(ev[i][5]) for i in range(K)]) if dec else None
    gt_ms = np.array([ev[i][6].elapsed_time(ev[i][7]) for i in range(K)]) if gated else None
    bw_ms = np.array([ev[i][8].elapsed_time(ev[i][9]) for i in range(K)]) if bwd else None
    log(f"[bench] prefill ms: mean {pf_ms.mean():.4f} min {pf_ms.min():.4f} "
        f"max {pf_ms.max():.4f}")

    pf_s = float(pf_ms.mean()) / 1e3
    alg_b = prefill_bytes(tokens, wl.H, wl.dk, wl.dv, n_seqs, S0 is not None)
    alg_f = prefill_flops(tokens, wl.H, wl.dk, wl.dv)
    achieved = alg_b / pf_s / 1e9
    out = {
        "metric": "KDA prefill tokens/s (H=32,d=128) + decode state GB/s, 1xMI355X, % roofline",
        "value": tokens / pf_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {n_seqs} seqs x "
                               f"{tokens // n_seqs if equal else 'varlen'} tokens, H={wl.H}, "
                               f"d_k=d_v={wl.dk}, bf16 q/k/v/o, fp32 g/beta/state, "
                               f"S0={'given' if S0 is not None else 'zero'}, S_T returned",
                   "tokens": tokens, "n_seqs": n_seqs, "H": wl.H, "d_k": wl.dk, "d_v": wl.dv,
                   "chunk": 16,
                   "scan_depth": scan_depth,
                   "split_workspace_bytes": int(ws_bytes),
                   "decode_workload": "256 seqs x 64 heads, d=128, fp32 state in place"
                   if dec else None},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None,
                     "kernel": "kda_prefill_kernel", "alg_bytes_per_launch": alg_b,
                     "launch_ms": pf_s * 1e3,
                     "mfma_tflops": alg_f / pf_s / 1e12,
                     "mfma_frac": alg_f / pf_s / 1e12 / BF16_PEAK_TFLOPS},
    }
    attach_counters(out["roofline"], args.workload, "prefill")
    if gated:
        gt_s = float(gt_ms.mean()) / 1e3
        gb = gated_prefill_bytes(tokens, wl.H, wl.dk, wl.dv, n_seqs)
        out["gated_prefill"] = {
            "workload": "the prefill workload from raw q/k, gate pre-activation z and beta "
                        "pre-activation b (bf16), A_log = 0: gate, beta and L2 norms in-kernel",
            "launch_ms": gt_s * 1e3, "tokens_per_s": tokens / gt_s,
            "roofline": {"bound": "hbm", "achieved": gb / gt_s / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": gb / gt_s / 1e9 / HBM_PEAK_GBS,
                         "kernel": "kda_prefill_kernel (gated)", "alg_bytes_per_launch": gb}}
        attach_counters(out["gated_prefill"]["roofline"], args.workload, "prefill_gated")
    if bwd:
        bw_s = float(bw_ms.mean()) / 1e3
        bb = backward_bytes(tokens, wl.H, wl.dk, wl.dv, n_seqs, S0 is not None)
        out["backward"] = {
            "workload": "gradients of the prefill workload (dq, dk, dv, dg, dbeta, dS0, fp32) "
                        "from seeded bf16 dO and fp32 dS_T: checkpointing forward, reverse "
                        "sweep and per-chunk finisher, timed as one call",
            "launch_ms": bw_s * 1e3, "tokens_per_s": tokens / bw_s,
            "roofline": {"bound": "hbm", "achieved": bb / bw_s / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": bb / bw_s / 1e9 / HBM_PEAK_GBS,
                         "kernel": "kda_bwd_chunked (3 kernels)", "alg_bytes_per_launch": bb}}
        attach_counters_sum(out["backward"]["roofline"], args.workload,
                            ("prefill_ckpt", "bwd_sweep_mfma", "bwd_chunk"))
    if dec:
        dw = WORKLOADS["decode"]
        st_b, all_b = decode_bytes(dw.n_seqs, dw.H, dw.dk, dw.dv)
        dc_s = float(dc_ms.mean()) / 1e3
        out["decode"] = {"state_GBps": st_b / dc_s / 1e9, "launch_ms": dc_s * 1e3,
                         "tokens_per_s": dw.n_seqs / dc_s,
                         "roofline": {"bound": "hbm", "achieved": all_b / dc_s / 1e9,
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": all_b / dc_s / 1e9 / HBM_PEAK_GBS,
                                      "kernel": "kda_decode_kernel",
                                      "alg_bytes_per_launch": all_b}}
        attach_counters(out["decode"]["roofline"], args.workload, "decode")
        sst_b, sall_b = spec_bytes(dw.n_seqs, dw.H, dw.dk, dw.dv, SPEC_K, SPEC_K)
        sp_s = float(sp_ms.mean()) / 1e3
        out["spec_decode"] = {
            "workload": f"{dw.n_seqs} seqs x {dw.H} heads, d=128: commit of {SPEC_K} previous "
                        f"drafts (seeded acceptance 0..{SPEC_K}) + verify of {SPEC_K} new drafts",
            "launch_ms": sp_s * 1e3, "state_GBps": sst_b / sp_s / 1e9,
            "draft_tokens_per_s": dw.n_seqs * SPEC_K / sp_s,
            "roofline": {"bound": "hbm", "achieved": sall_b / sp_s / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": sall_b / sp_s / 1e9 / HBM_PEAK_GBS,
                         "kernel": "kda_spec_kernel", "alg_bytes_per_launch": sall_b}}
        attach_counters(out["spec_decode"]["roofline"], args.workload, "spec")
    if not args.no_cpu:
        threads = min(16, os.cpu_count() or 1)
        out["cpu_baseline"] = cpu_baseline(threads)
        if args.workload == "prefill":
            out["cpu_baseline"]["gpu_speedup"] = out["value"] / out["cpu_baseline"]["value"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
