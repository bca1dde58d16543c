"""Turn rocprofv3 output of `bench.py` runs into the short summaries kept
under profiles/.

  python profile_summary.py stats <trace_dir> <out.md> "<command>"
      kernel-trace statistics (rocprofv3 --kernel-trace --stats
      --output-format csv) as a table
  python profile_summary.py pmc <out.json> <workload> <copy_mib> "<commands>" \\
                                <fetch_dir> <write_dir> [<sq_dir>]
      per kernel of the run: HBM bytes per dispatch from one FETCH_SIZE and
      one WRITE_SIZE pass, each scaled by what the same counter reads for the
      plain device copy of <copy_mib> MiB that `bench.py --calib-copy-mib`
      runs; with <sq_dir>, the SQ pass of SQ_COUNTERS below turned into
      matrix-core busy, vector-ALU busy and LDS bank-conflict fractions

The JSON records, per kernel, the hash of the sources that kernel is built
from; bench.py uses a kernel's figures only while that hash matches and
only for the record's own workload.
"""
import csv
import glob
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "gated_delta_rule_95_amd", "csrc")

# MI355X: 256 compute units, 4 SIMDs each
CU_NUM, SIMD_NUM = 256, 1024
# GRBM_GUI_ACTIVE counts GPU cycles in each XCD's graphics block, and
# rocprofv3 reports the sum over the XCDs of the chip (one row per dispatch):
# the kernel's duration in cycles is that sum over XCD_NUM
XCD_NUM = 8
SQ_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_LDS_BANK_CONFLICT",
               "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
               "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]


def kernel_class(name: str):
    """Which of the library's kernels (or the calibration copy) a dispatch is."""
    if "copyBuffer" in name:
        return "copy"
    if "kda_prefill_kernel" in name:
        # the last two template arguments: gated prologue, checkpointing
        m = re.search(r"Lb([01])ELb([01])E", name)
        if m and m.group(2) == "1":
            return "prefill_ckpt"
        return "prefill_gated" if m and m.group(1) == "1" else "prefill"
    for key in ("kda_decode_kernel", "kda_spec_kernel", "kda_seg_scan_kernel",
                "kda_seg_correct_kernel", "kda_bwd_sweep_mfma", "kda_bwd_sweep",
                "kda_bwd_finish", "kda_bwd_chunk"):
        if key in name:
            return key.replace("kda_", "").replace("_kernel", "")
    return None


# the sources each kernel class is built from (every kernel also includes
# the shared device and launch headers)
_PF = ("kda_prefill.hip", "kda_chunk.h")
_BW = ("kda_backward.hip", "kda_chunk.h")
KERNEL_SOURCE = {"prefill": _PF, "prefill_gated": _PF, "prefill_ckpt": _PF,
                 "seg_scan": _PF, "seg_correct": _PF,
                 "decode": ("kda_decode.hip",), "spec": ("kda_spec.hip",),
                 "bwd_sweep": _BW, "bwd_finish": _BW, "bwd_sweep_mfma": _BW,
                 "bwd_chunk": _BW}
SHARED_HEADERS = ("kda_device.h", "kda_launch.h")


def source_hash(cls: str) -> str:
    """sha256 (16 hex digits) over the sources kernel class `cls` is built
    from: its own files and the shared headers."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCE[cls] + SHARED_HEADERS:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _rows(d, pattern):
    out = []
    for f in sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True)):
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def stats(trace_dir, out_md, command):
    rows = _rows(trace_dir, "*kernel_stats.csv")
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    lines = ["# rocprofv3 kernel statistics", "", "Command (from the repository root on the "
             "GPU):", "", "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | share |",
             "|---|---|---|---|---|---|"]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    for r in rows:
        name = r["Name"]
        cls = kernel_class(name)
        short = (cls + ": " if cls else "") + name.split("(")[0][:80]
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counters(d):
    """{(kernel class, dispatch id): {counter: value summed over instances}}."""
    acc = {}
    for r in _rows(d, "*counter_collection.csv"):
        cls = kernel_class(r["Kernel_Name"])
        if cls is None:
            continue
        key = (cls, r["Dispatch_Id"])
        c = acc.setdefault(key, {})
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return acc


def _median(vals):
    vals = sorted(vals)
    return vals[len(vals) // 2] if vals else None


def _per_class(acc, counter):
    per = {}
    for (cls, _), c in acc.items():
        if counter in c:
            per.setdefault(cls, []).append(c[counter])
    return {cls: _median(v) for cls, v in per.items()}


def pmc(out_json, workload, copy_mib, commands, fetch_dir, write_dir, sq_dir=None):
    copy_bytes = int(copy_mib) * (1 << 20)
    fe = _per_class(_counters(fetch_dir), "FETCH_SIZE")
    wr = _per_class(_counters(write_dir), "WRITE_SIZE")
    if "copy" not in fe or "copy" not in wr:
        raise SystemExit("the calibration copy is missing from the counter output")
    rf, rw = copy_bytes / (fe["copy"] * 1024), copy_bytes / (wr["copy"] * 1024)
    rec = {"workload": workload,
           "copy_bytes": copy_bytes, "copy_fetch_raw": fe["copy"] * 1024,
           "copy_write_raw": wr["copy"] * 1024, "fetch_scale": rf, "write_scale": rw,
           "commands": commands, "kernels": {}}
    for cls in sorted(set(fe) | set(wr)):
        if cls == "copy":
            continue
        k = rec["kernels"].setdefault(cls, {"source_sha256_16": source_hash(cls)})
        if cls in fe:
            k["fetch_bytes"] = fe[cls] * 1024 * rf
        if cls in wr:
            k["write_bytes"] = wr[cls] * 1024 * rw
        if cls in fe and cls in wr:
            k["hbm_bytes_per_dispatch"] = k["fetch_bytes"] + k["write_bytes"]
    if sq_dir:
        acc = _counters(sq_dir)
        per = {name: _per_class(acc, name) for name in SQ_COUNTERS}
        for cls in per["GRBM_GUI_ACTIVE"]:
            if cls == "copy":
                continue
            gui = per["GRBM_GUI_ACTIVE"][cls]
            cycles = gui / XCD_NUM if gui else None
            k = rec["kernels"].setdefault(cls, {"source_sha256_16": source_hash(cls)})
            raw = {name: per[name].get(cls) for name in SQ_COUNTERS}
            k["sq_raw"] = raw
            # rocprofv3's derived metrics: MfmaUtil, VALUBusy, LDSBankConflict
            if cycles:
                k["duration_cycles"] = cycles
                k["mfma_busy_pct"] = 100.0 * (raw["SQ_VALU_MFMA_BUSY_CYCLES"] or 0) / (cycles * SIMD_NUM)
                k["valu_busy_pct"] = 100.0 * (raw["SQ_ACTIVE_INST_VALU"] or 0) * 4 / SIMD_NUM / cycles
                k["lds_bank_conflict_pct"] = 100.0 * (raw["SQ_LDS_BANK_CONFLICT"] or 0) / CU_NUM / cycles
            if raw["SQ_INSTS_VALU_MFMA_MOPS_BF16"] is not None:
                k["mfma_bf16_flops"] = raw["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        rec["sq_counters"] = SQ_COUNTERS
        rec["sq_note"] = ("The SQ counters and GRBM_GUI_ACTIVE are chip-wide sums per "
                          "dispatch; GRBM_GUI_ACTIVE sums the XCDs' cycle counts, so the "
                          f"duration in cycles is it over XCD_NUM = {XCD_NUM}.  The "
                          "percentages are rocprofv3's MfmaUtil, VALUBusy and "
                          "LDSBankConflict expressions on that duration, with "
                          f"CU_NUM = {CU_NUM}, SIMD_NUM = {SIMD_NUM}")
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "stats" and len(sys.argv) == 5:
        stats(*sys.argv[2:])
    elif len(sys.argv) >= 2 and sys.argv[1] == "pmc" and len(sys.argv) in (8, 9):
        pmc(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
