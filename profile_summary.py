"""Turn rocprofv3 output of `bench.py` runs into the short summaries kept
under profiles/.

  python profile_summary.py stats <trace_dir> <out.md> "<command>"
      kernel-trace statistics (rocprofv3 --kernel-trace --stats) as a table
  python profile_summary.py pmc <fetch_dir> <write_dir> <copy_mib> <out.json> "<commands>"
      HBM bytes per prefill launch from one FETCH_SIZE and one WRITE_SIZE
      pass over the default bench workload (prefill), each scaled by what the
      same counter reads for the plain device copy of <copy_mib> MiB that
      `bench.py --calib-copy-mib` runs

The JSON records the hash of the kernel sources it was taken on; bench.py
reports the traffic only while that hash matches.
"""
import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
PREFILL = "kda_prefill_kernel"


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
             "GPU box):", "", "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | share |",
             "|---|---|---|---|---|---|"]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    for r in rows:
        name = r["Name"]
        short = name.split("(")[0][:90]
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter(d, counter):
    """{kernel name: [value per dispatch]} for one counter (KiB per dispatch)."""
    per = {}
    acc = {}
    for r in _rows(d, "*counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    for (name, _), v in acc.items():
        per.setdefault(name, []).append(v)
    return per


def _pick(per, pred):
    vals = [v for name, vs in per.items() if pred(name) for v in vs]
    if not vals:
        raise SystemExit("kernel not found in counter output")
    vals.sort()
    return vals[len(vals) // 2]


def pmc(fetch_dir, write_dir, copy_mib, out_json, commands):
    sys.path.insert(0, ROOT)
    from bench import source_hash
    copy_bytes = int(copy_mib) * (1 << 20)
    is_copy = lambda n: "copyBuffer" in n                             # noqa: E731
    is_pf = lambda n: PREFILL in n                                   # noqa: E731
    fe, wr = _counter(fetch_dir, "FETCH_SIZE"), _counter(write_dir, "WRITE_SIZE")
    cf, cw = _pick(fe, is_copy) * 1024, _pick(wr, is_copy) * 1024
    pf, pw = _pick(fe, is_pf) * 1024, _pick(wr, is_pf) * 1024
    rf, rw = copy_bytes / cf, copy_bytes / cw
    rec = {"kernel": PREFILL, "workload": "prefill",
           "fetch_bytes_raw": pf, "write_bytes_raw": pw,
           "copy_bytes": copy_bytes, "copy_fetch_raw": cf, "copy_write_raw": cw,
           "fetch_scale": rf, "write_scale": rw,
           "hbm_bytes_per_launch": pf * rf + pw * rw,
           "kernel_source_sha256_16": source_hash(),
           "commands": commands}
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "stats" and len(sys.argv) == 5:
        stats(*sys.argv[2:])
    elif len(sys.argv) >= 2 and sys.argv[1] == "pmc" and len(sys.argv) == 7:
        pmc(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
