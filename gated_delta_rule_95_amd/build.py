"""Build libkda.so (HIP, gfx950) in-tree with hipcc.

    python -m gated_delta_rule_95_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled (-packed-fp32-ops), and linked into one shared library
next to this file.  The C-ABI declarations are in include/kda.h.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkda.so")
ARCH = "gfx950"
SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_prefill.hip", "kda_noalloc.hip",
           "kda_spec.hip", "kda_backward.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkda)")


def flags() -> list:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + INCLUDE, "-I" + CSRC]


def build(verbose: bool = False, jobs: int = 4) -> str:
    cc = hipcc()
    tmpdir = tempfile.mkdtemp(prefix="kda_build_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            cmd = [cc] + flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
            while len([p for _, p in procs if p.poll() is None]) >= jobs:
                procs[0][1].wait()
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            out = "\n".join(line for line in out.splitlines()
                            if "packed-fp32-ops' is not a recognized feature" not in line)
            if out.strip() and (verbose or p.returncode):
                print(out, file=sys.stderr)
            if p.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError("hipcc failed for: " + ", ".join(failed))
        tmp_lib = LIB + ".tmp%d" % os.getpid()
        cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp_lib] + objs
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
