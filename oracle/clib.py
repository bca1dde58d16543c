"""ctypes wrapper of the plain-C fp64 oracle (kda_oracle.c) -- test
infrastructure only.  Builds ``liboracle.so`` with gcc on first use if it is
not there (``__graft_entry__.build()`` also builds it)."""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "kda_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no fast-math)."""
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-march=x86-64-v3", "-fno-fast-math",
           "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB):
                build()
            lib = ctypes.CDLL(LIB)
            f = lib.kda_oracle_fwd
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 4 + \
                [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
            h = lib.kda_oracle_head
            h.restype = None
            h.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 7
            b = lib.kda_oracle_vjp
            b.restype = ctypes.c_int
            b.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 4 + [ctypes.c_void_p] * 6 + \
                [ctypes.c_int]
            _lib = lib
    return _lib


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _p(a):
    return None if a is None else a.ctypes.data


def fwd(q, k, v, g, beta, cu_seqlens, S0=None, want_o: bool = True,
        threads: int = 0) -> Tuple[Optional[np.ndarray], np.ndarray, int]:
    """Packed varlen batch in fp64.  q, k, g [N, H, dk]; v [N, H, dv];
    beta [N, H]; S0 [n_seqs, H, dk, dv] or None; cu_seqlens int [n_seqs+1].
    Returns (o [N, H, dv] or None, S_T [n_seqs, H, dk, dv], threads used)."""
    lib = _load()
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    N, H, dk = q.shape
    dv = v.shape[-1]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    ns = len(cu) - 1
    s0 = None if S0 is None else _f32(S0)
    o = np.zeros((N, H, dv)) if want_o else None
    ST = np.zeros((ns, H, dk, dv))
    used = lib.kda_oracle_fwd(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(s0), _p(cu),
                              ns, H, dk, dv, _p(o), _p(ST), int(threads))
    return o, ST, used


def head(q, k, v, g, beta, S0=None, want_o: bool = True
         ) -> Tuple[Optional[np.ndarray], np.ndarray]:
    """Single chain with contiguous arrays: q, k, g [T, dk]; v [T, dv];
    beta [T]; S0 [dk, dv].  Releases the GIL while it runs."""
    lib = _load()
    q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
    T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64, copy=True, order="C")
    o = np.zeros((T, dv)) if want_o else None
    lib.kda_oracle_head(T, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta), _p(S), _p(o))
    return o, S


def vjp(q, k, v, g, beta, dO, cu_seqlens, S0=None, dST=None, threads: int = 0):
    """Reverse-mode gradients of the packed varlen batch in fp64 (every
    sequence independent, its own S0 and dS_T).  Shapes as in fwd(); dO
    [N, H, dv]; dST [n_seqs, H, dk, dv] or None.  Returns dq, dk, dv, dg,
    dbeta, dS0 (fp64) and the threads used.  Each thread keeps every state of
    the longest sequence (T + 1 states of dk x dv doubles)."""
    lib = _load()
    q, k, v, g, beta, dO = (_f32(x) for x in (q, k, v, g, beta, dO))
    N, H, dk = q.shape
    dv = v.shape[-1]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    ns = len(cu) - 1
    s0 = None if S0 is None else _f32(S0)
    dst = None if dST is None else _f32(dST)
    dq, dkk, dg = (np.zeros((N, H, dk)) for _ in range(3))
    dvv = np.zeros((N, H, dv))
    db = np.zeros((N, H))
    dS0 = np.zeros((ns, H, dk, dv))
    used = lib.kda_oracle_vjp(_p(q), _p(k), _p(v), _p(g), _p(beta), _p(s0), _p(dO), _p(dst),
                              _p(cu), ns, H, dk, dv, _p(dq), _p(dkk), _p(dvv), _p(dg), _p(db),
                              _p(dS0), int(threads))
    if used < 0:
        raise MemoryError("kda_oracle_vjp: state buffer allocation failed")
    return dq, dkk, dvv, dg, db, dS0, used
