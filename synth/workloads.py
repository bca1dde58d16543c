"""Workload shapes, value distributions and the seeded generators.

Distributions (the second argument of N(0, s) is the standard deviation):
  q, k : N(0, 1) per element, L2-normalised per token in fp32, then (bf16
         workloads) rounded to bfloat16 with round-to-nearest-even.
  v    : N(0, 1)  (bf16-rounded for bf16 workloads).
  g    : log-decay  -5 * sigmoid(N(0, g_sigma)), fp32, per key channel, so
         every g lies in (-5, 0); the stress workload puts half of the heads
         at U[-5, -4.9], next to the lower bound.
  beta : sigmoid(N(0, 1)), fp32; the stress workload forces beta = 1 on a
         seeded 10 % of token positions (the same positions for every head).
  S0   : N(0, s0_sigma) fp32 per element when the workload carries a state.

The gate lower bound of -5 is the one the K3 pages give for KDA (K3-on-TPU
essay, blog.higcp.com, section on KDA + Gated MLA, "lower-bounded decay").
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

SEED_BASE = 0x4B4441

# tensor ids inside a (sequence, head) stream family
_Q, _K, _V, _G, _BETA, _S0, _BMASK, _LEN = 1, 2, 3, 4, 5, 6, 7, 8


@dataclass(frozen=True)
class Workload:
    name: str
    seed_index: int
    H: int
    dk: int
    dv: int
    dtype: str                      # "f32" or "bf16" (q, k, v and o)
    n_seqs: int = 1
    seqlen: Optional[int] = None    # equal-length sequences; None => varlen
    varlen_target_tokens: Optional[int] = None  # keep drawing until reached
    g_sigma: float = 1.0
    s0_sigma: Optional[float] = None
    stress: bool = False
    decode: bool = False
    chunk: int = 16
    notes: str = ""

    @property
    def seed(self) -> int:
        return SEED_BASE + self.seed_index


WORKLOADS: Dict[str, Workload] = {
    # B=1, H=1, T=64, d_k=d_v=16, fp32, chunk 16, S0 = 0
    "tiny": Workload("tiny", 0, H=1, dk=16, dv=16, dtype="f32", n_seqs=1,
                     seqlen=64, g_sigma=1.0),
    # B=4, T=4096, H=32, d=128, bf16 q/k/v, g = -5 sigmoid(N(0,1.5)), S0 = 0
    "prefill": Workload("prefill", 1, H=32, dk=128, dv=128, dtype="bf16",
                        n_seqs=4, seqlen=4096, g_sigma=1.5),
    # B=1, T=65536, H=64, d=128, bf16, g and beta drawn as in "tiny",
    # S0 ~ N(0, 0.02), S_T returned for carry-over
    "long_prefill": Workload("long_prefill", 2, H=64, dk=128, dv=128,
                             dtype="bf16", n_seqs=1, seqlen=65536,
                             g_sigma=1.0, s0_sigma=0.02),
    # 256 sequences x 64 heads, one token each, S ~ N(0, 0.05) in place
    "decode": Workload("decode", 3, H=64, dk=128, dv=128, dtype="bf16",
                       n_seqs=256, seqlen=1, g_sigma=1.0, s0_sigma=0.05,
                       decode=True),
    # 64 sequences, log-uniform lengths in [128, 32768], H=32, d=128, bf16,
    # decay stress on half of the heads, beta = 1 on 10 % of tokens, keys
    # repeated inside every 16-token tile
    "varlen": Workload("varlen", 4, H=32, dk=128, dv=128, dtype="bf16",
                       n_seqs=64, seqlen=None, g_sigma=1.5, stress=True),
    # same distributions, log-uniform lengths drawn until 2^20 tokens
    "varlen_1m": Workload("varlen_1m", 5, H=32, dk=128, dv=128, dtype="bf16",
                          n_seqs=0, seqlen=None, varlen_target_tokens=1 << 20,
                          g_sigma=1.5, stress=True),
}


# ----------------------------------------------------------------------------
# bfloat16 helpers (round-to-nearest-even on the fp32 bit pattern)
# ----------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value, returned as fp32."""
    return bf16_bits_to_f32(bf16_bits(x))


# ----------------------------------------------------------------------------
# streams
# ----------------------------------------------------------------------------
def _rng(wl: Workload, *key: int) -> np.random.Generator:
    ss = np.random.SeedSequence(wl.seed, spawn_key=tuple(int(k) for k in key))
    return np.random.Generator(np.random.PCG64(ss))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


def seq_lengths(wl: Workload) -> np.ndarray:
    """Sequence lengths of a workload (int64)."""
    if wl.seqlen is not None:
        return np.full(wl.n_seqs, wl.seqlen, dtype=np.int64)
    rng = _rng(wl, 0xFFFF, _LEN)
    if wl.varlen_target_tokens is None:
        u = rng.random(wl.n_seqs)
        return np.rint(128.0 * 256.0 ** u).astype(np.int64)
    out, total = [], 0
    while total < wl.varlen_target_tokens:
        n = int(np.rint(128.0 * 256.0 ** rng.random()))
        n = min(n, wl.varlen_target_tokens - total)
        out.append(n)
        total += n
    return np.asarray(out, dtype=np.int64)


def cu_seqlens(lengths: np.ndarray) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    if cu[-1] >= 2**31:
        raise ValueError("total token count does not fit int32")
    return cu.astype(np.int32)


def _maybe_bf16(wl: Workload, x: np.ndarray) -> np.ndarray:
    return round_bf16(x) if wl.dtype == "bf16" else x.astype(np.float32)


def head_inputs(wl: Workload, n: int, h: int, T: int, raw: bool = False) -> Dict[str, np.ndarray]:
    """Inputs of sequence n, head h (T tokens) as fp32 arrays.

    q, k : [T, dk]   v : [T, dv]   g : [T, dk]   beta : [T]
    s0   : [dk, dv] or absent.   Values of bf16 workloads are bf16-exact.

    raw=True returns the same streams' draws before the L2 normalisation
    and the sigmoids: q, k (unnormalised), v, z : [T, dk] (the N(0, g_sigma)
    draw), b : [T] (the N(0, 1) draw), all in the workload's dtype, for the
    fused-prologue entry point with A_log = 0 (then g = -5 sigmoid(z) and
    beta = sigmoid(b) are the workload's distributions).  Not for the
    stress workloads.
    """
    dk, dv = wl.dk, wl.dv
    if raw:
        if wl.stress:
            raise ValueError("raw inputs are not defined for the stress workloads")
        q = _rng(wl, n, h, _Q).standard_normal((T, dk), dtype=np.float32)
        k = _rng(wl, n, h, _K).standard_normal((T, dk), dtype=np.float32)
        v = _rng(wl, n, h, _V).standard_normal((T, dv), dtype=np.float32)
        z = _rng(wl, n, h, _G).standard_normal((T, dk), dtype=np.float32) * \
            np.float32(wl.g_sigma)
        b = _rng(wl, n, h, _BETA).standard_normal(T, dtype=np.float32)
        out = {key: _maybe_bf16(wl, x) for key, x in
               (("q", q), ("k", k), ("v", v), ("z", z), ("b", b))}
        if wl.s0_sigma is not None:
            out["s0"] = (_rng(wl, n, h, _S0).standard_normal((dk, dv), dtype=np.float32)
                         * np.float32(wl.s0_sigma))
        return out
    q = _unit_rows(_rng(wl, n, h, _Q).standard_normal((T, dk), dtype=np.float32))
    k = _unit_rows(_rng(wl, n, h, _K).standard_normal((T, dk), dtype=np.float32))
    v = _rng(wl, n, h, _V).standard_normal((T, dv), dtype=np.float32)
    rg = _rng(wl, n, h, _G)
    if wl.stress and h < wl.H // 2:
        g = rg.uniform(-5.0, -4.9, size=(T, dk)).astype(np.float32)
    else:
        g = (np.float32(-5.0) * _sigmoid(
            rg.standard_normal((T, dk), dtype=np.float32) * np.float32(wl.g_sigma)))
    beta = _sigmoid(_rng(wl, n, h, _BETA).standard_normal(T, dtype=np.float32))
    if wl.stress:
        mask = _rng(wl, n, 0xFFFF, _BMASK).random(T) < 0.1
        beta = np.where(mask, np.float32(1.0), beta).astype(np.float32)
        # repeat keys inside every 16-token tile aligned to the sequence start:
        # position p with p % 16 >= 8 takes the key of p - 8
        dst = np.nonzero(np.arange(T) % 16 >= 8)[0]
        k[dst] = k[dst - 8]
    out = {"q": _maybe_bf16(wl, q), "k": _maybe_bf16(wl, k),
           "v": _maybe_bf16(wl, v), "g": g.astype(np.float32),
           "beta": beta.astype(np.float32)}
    if wl.s0_sigma is not None:
        out["s0"] = (_rng(wl, n, h, _S0).standard_normal((dk, dv), dtype=np.float32)
                     * np.float32(wl.s0_sigma))
    return out


def decode_head_inputs(wl: Workload, n: int, h: int) -> Dict[str, np.ndarray]:
    """One decode token of sequence n, head h: q, k [dk], v [dv], g [dk],
    beta scalar array, and the incoming state S [dk, dv]."""
    d = head_inputs(wl, n, h, 1)
    return {"q": d["q"][0], "k": d["k"][0], "v": d["v"][0], "g": d["g"][0],
            "beta": d["beta"][:1], "S": d["s0"]}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def batch_inputs(wl: Workload, lengths: Optional[np.ndarray] = None,
                 threads: Optional[int] = None,
                 seqs: Optional[range] = None, raw: bool = False) -> Dict[str, np.ndarray]:
    """Whole packed batch, token-major, fp32 arrays (bf16-exact for bf16).

    Returns q, k [N, H, dk]; v [N, H, dv]; g [N, H, dk]; beta [N, H];
    s0 [n_seqs, H, dk, dv] (only if the workload has a state);
    cu_seqlens int32 [n_seqs + 1]; lengths int64 [n_seqs].

    With `seqs` (a range of sequence indices) only those sequences are
    generated, packed back to back from token 0 (cu_seqlens local to the
    group); every value equals the one the whole batch holds for them.
    """
    if lengths is None:
        lengths = seq_lengths(wl)
    lengths = np.asarray(lengths, np.int64)
    first = 0
    if seqs is not None:
        first = seqs.start
        lengths = lengths[seqs.start:seqs.stop]
    cu = cu_seqlens(lengths)
    N, H, dk, dv = int(cu[-1]), wl.H, wl.dk, wl.dv
    ns = len(lengths)
    gk, bk = ("z", "b") if raw else ("g", "beta")
    out = {
        "q": np.empty((N, H, dk), np.float32), "k": np.empty((N, H, dk), np.float32),
        "v": np.empty((N, H, dv), np.float32), gk: np.empty((N, H, dk), np.float32),
        bk: np.empty((N, H), np.float32),
    }
    if wl.s0_sigma is not None:
        out["s0"] = np.empty((ns, H, dk, dv), np.float32)

    def work(nh):
        n, h = nh
        a, b = int(cu[n]), int(cu[n + 1])
        d = head_inputs(wl, first + n, h, b - a, raw=raw)
        for key in ("q", "k", "v", gk):
            out[key][a:b, h] = d[key]
        out[bk][a:b, h] = d[bk]
        if "s0" in d:
            out["s0"][n, h] = d["s0"]

    pairs = [(n, h) for n in range(ns) for h in range(H)]
    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(work, pairs))
    out["cu_seqlens"] = cu
    out["lengths"] = np.asarray(lengths, np.int64)
    return out


def decode_batch_inputs(wl: Workload, threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Decode batch: q, k, g [N, H, dk]; v [N, H, dv]; beta [N, H];
    S [N, H, dk, dv] fp32."""
    N, H, dk, dv = wl.n_seqs, wl.H, wl.dk, wl.dv
    out = {"q": np.empty((N, H, dk), np.float32), "k": np.empty((N, H, dk), np.float32),
           "v": np.empty((N, H, dv), np.float32), "g": np.empty((N, H, dk), np.float32),
           "beta": np.empty((N, H), np.float32), "S": np.empty((N, H, dk, dv), np.float32)}

    def work(nh):
        n, h = nh
        d = decode_head_inputs(wl, n, h)
        for key in ("q", "k", "v", "g", "S"):
            out[key][n, h] = d[key]
        out["beta"][n, h] = d["beta"][0]

    pairs = [(n, h) for n in range(N) for h in range(H)]
    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(work, pairs))
    return out


def draft_batch_inputs(wl: Workload, K: int, stream: int,
                       threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """K drafted tokens for each of the decode workload's sequences, drawn
    with the workload's distributions: q, k, g [N, K, H, dk]; v [N, K, H,
    dv]; beta [N, K, H].  `stream` (>= 1) selects an independent set of
    streams (sequence index n + stream * N), e.g. one for a step's drafts
    and another for the previous step's."""
    N, H, dk, dv = wl.n_seqs, wl.H, wl.dk, wl.dv
    out = {"q": np.empty((N, K, H, dk), np.float32), "k": np.empty((N, K, H, dk), np.float32),
           "v": np.empty((N, K, H, dv), np.float32), "g": np.empty((N, K, H, dk), np.float32),
           "beta": np.empty((N, K, H), np.float32)}

    def work(nh):
        n, h = nh
        d = head_inputs(wl, n + stream * N, h, K)
        for key in ("q", "k", "v", "g"):
            out[key][n, :, h] = d[key]
        out["beta"][n, :, h] = d["beta"]

    pairs = [(n, h) for n in range(N) for h in range(H)]
    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(work, pairs))
    return out


def describe(wl: Workload) -> str:
    L = seq_lengths(wl)
    return (f"{wl.name}: seqs={len(L)} tokens={int(L.sum())} H={wl.H} dk={wl.dk} "
            f"dv={wl.dv} dtype={wl.dtype}")
