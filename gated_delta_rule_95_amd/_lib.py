"""ctypes binding of libkda.so (the C ABI in include/kda.h).

Argument marshalling only: every step of KDA runs in the library's HIP
kernels.  There is no fallback: if libkda.so is missing or cannot be loaded
the import of the entry points raises.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "kda.h")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP = 0, 1, 2, 3
KDA_F32, KDA_BF16 = 0, 1

_lock = threading.Lock()
_lib = None


class KDAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libkda.so (built by gated_delta_rule_95_amd.build) and declare
    the argument types of every entry point."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m gated_delta_rule_95_amd.build` "
                "(or __graft_entry__.build()) first. There is no CPU fallback.")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        SZ = ctypes.c_size_t
        lib.kda_fwd_chunked.restype = ctypes.c_int
        lib.kda_fwd_chunked.argtypes = [P, P, P, P, P, P, P, I32, I64, I32, I32, I32,
                                        ctypes.c_int, ctypes.c_int, P, P, P, SZ, P]
        lib.kda_fwd_chunked_gated.restype = ctypes.c_int
        lib.kda_fwd_chunked_gated.argtypes = [P, P, P, P, P, P, P, P, I32, I64, I32, I32, I32,
                                              ctypes.c_int, ctypes.c_int, P, P, P, SZ, P]
        lib.kda_fwd_chunked_noalloc.restype = ctypes.c_int
        lib.kda_fwd_chunked_noalloc.argtypes = [P, P, P, P, P, P, P, I32, I64, I32, I32, I32,
                                                ctypes.c_int, ctypes.c_int, P, P, P]
        lib.kda_fwd_workspace_bytes.restype = SZ
        lib.kda_fwd_workspace_bytes.argtypes = [I32, I64, I32, I32, I32, ctypes.c_int]
        lib.kda_decode_step.restype = ctypes.c_int
        lib.kda_decode_step.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32,
                                        ctypes.c_int, ctypes.c_int, P, P]
        lib.kda_decode_verify.restype = ctypes.c_int
        lib.kda_decode_verify.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32,
                                          ctypes.c_int, ctypes.c_int, P, P]
        lib.kda_decode_commit.restype = ctypes.c_int
        lib.kda_decode_commit.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32,
                                          ctypes.c_int, P]
        lib.kda_decode_spec.restype = ctypes.c_int
        lib.kda_decode_spec.argtypes = [P, P, P, P, P, I32, P, P, P, P, P, I32, P, I32, I32,
                                        I32, I32, ctypes.c_int, ctypes.c_int, P, P]
        lib.kda_bwd_workspace_bytes.restype = SZ
        lib.kda_bwd_workspace_bytes.argtypes = [I32, I64, I32, I32, I32]
        lib.kda_bwd_chunked.restype = ctypes.c_int
        lib.kda_bwd_chunked.argtypes = [P, P, P, P, P, P, P, I32, I64, I32, I32, I32,
                                        ctypes.c_int, P, P, P, P, P, P, P, P, P, SZ, P]
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_status_string.argtypes = [ctypes.c_int]
        lib.kda_last_error.restype = ctypes.c_char_p
        lib.kda_last_error.argtypes = []
        lib.kda_version.restype = ctypes.c_char_p
        lib.kda_version.argtypes = []
        _lib = lib
        return lib


def status_string(s: int) -> str:
    return load().kda_status_string(int(s)).decode()


def last_error() -> str:
    return load().kda_last_error().decode()


def version() -> str:
    return load().kda_version().decode()


def check(status: int) -> None:
    if status != KDA_OK:
        raise KDAError(status, last_error())


def header_functions() -> list:
    """Names of the functions include/kda.h declares."""
    with open(HEADER) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))
