"""Helpers shared by the GPU tests: move seeded synthetic batches to the
device, and compare a device result with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch


def err(x, ref) -> float:
    """max |x - ref| / rms(ref): the tolerance metric for o and S_T."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.max(np.abs(x - ref), initial=0.0))
    return float(np.max(np.abs(x - ref), initial=0.0)) / rms


def half_ulp_bf16(ref) -> np.ndarray:
    """Largest round-to-nearest error of storing |ref| in bfloat16."""
    a = np.abs(np.asarray(ref, np.float64))
    e = np.floor(np.log2(np.maximum(a, 1e-300)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def err_bf16_out(x, ref) -> float:
    """Tolerance metric for a bf16-stored output: the storage rounding of each
    element (at most half a bf16 ulp of the exact value) is allowed on top
    of the computation error, which is what is then measured."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    excess = np.maximum(np.abs(x - ref) - half_ulp_bf16(ref), 0.0)
    return float(np.max(excess, initial=0.0)) / (rms if rms else 1.0)


def to_dev(batch: dict, dtype: torch.dtype, dev="cuda") -> dict:
    """fp32 numpy batch (bf16-exact for bf16 workloads) -> device tensors."""
    out = {}
    for key in ("q", "k", "v"):
        out[key] = torch.from_numpy(batch[key]).to(dev).to(dtype).contiguous()
    for key in ("g", "beta"):
        out[key] = torch.from_numpy(batch[key]).to(dev).contiguous()
    for key in ("s0", "S"):
        if key in batch:
            out[key] = torch.from_numpy(batch[key]).to(dev).contiguous()
    if "cu_seqlens" in batch:
        out["cu_seqlens"] = torch.from_numpy(batch["cu_seqlens"].astype(np.int32)).to(dev)
    return out


def random_batch(seed, lengths, H, dk, dv, s0=True, gmin=-5.0, bf16=True):
    """Small packed batch with the workload distributions (for edge cases)."""
    from synth import round_bf16
    r = np.random.default_rng(seed)
    lengths = np.asarray(lengths, np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    N = int(cu[-1])

    def unit(x):
        return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)
    q = unit(r.standard_normal((N, H, dk)).astype(np.float32))
    k = unit(r.standard_normal((N, H, dk)).astype(np.float32))
    v = r.standard_normal((N, H, dv)).astype(np.float32)
    if bf16:
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    g = (gmin / (1.0 + np.exp(-r.standard_normal((N, H, dk)) * 1.5))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-r.standard_normal((N, H))))).astype(np.float32)
    out = {"q": q, "k": k, "v": v, "g": g, "beta": beta, "cu_seqlens": cu, "lengths": lengths}
    if s0:
        out["s0"] = (r.standard_normal((len(lengths), H, dk, dv)) * 0.5).astype(np.float32)
    return out
