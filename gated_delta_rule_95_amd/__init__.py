"""gated_delta_rule_95_amd -- Kimi Delta Attention (KDA) on MI355X.

Thin Python front of libkda.so (C ABI: include/kda.h).  PyTorch supplies
device memory and the current HIP stream; every step of KDA runs in the
library's hand-written gfx950 kernels.  Names follow the C ABI:

    kda_fwd_chunked(q, k, v, g, beta, S0=None, cu_seqlens=None, ...) -> (o, S_T)
    kda_fwd_chunked_gated(q, k, v, z, A_log, b, ...) -> (o, S_T)   (gate + q/k norm fused)
    kda_fwd_workspace_bytes(n_seqs, n_tokens, H, d_k, d_v, dtype) -> int
    kda_bwd_chunked(q, k, v, g, beta, dO, S0=None, dS_T=None, ...) -> (dq, dk, dv, dg, dbeta, dS0)
    kda_decode_step(q, k, v, g, beta, S, ...) -> o        (S updated in place)
    kda_decode_verify(q, k, v, g, beta, S, ...) -> o      (K drafts, S read only)
    kda_decode_commit(k, v, g, beta, n_accept, S)         (replay accepted, S in place)
    kda_decode_spec(q, k, v, g, beta, S, prev, n_accept) -> o   (both in one pass)
"""
from __future__ import annotations

from typing import Optional, Tuple, Union

import torch

from . import _lib
from ._lib import KDAError, KDA_BF16, KDA_F32, KDA_OK  # noqa: F401

__all__ = ["kda_fwd_chunked", "kda_fwd_chunked_gated", "kda_fwd_workspace_bytes",
           "kda_bwd_chunked", "kda_bwd_workspace_bytes",
           "kda_decode_step",
           "kda_decode_verify", "kda_decode_commit", "kda_decode_spec", "KDAError",
           "version", "library_path"]


def library_path() -> str:
    return _lib.LIB_PATH


def version() -> str:
    return _lib.version()


def _dt(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return KDA_BF16
    if t == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t}; KDA takes bfloat16 or float32 q/k/v")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def kda_fwd_workspace_bytes(n_seqs: int, n_tokens: int, H: int, d_k: int, d_v: int,
                            dtype: torch.dtype = torch.bfloat16) -> int:
    """Bytes of workspace with which kda_fwd_chunked may take the
    sequence-split path for these sizes on the current device (0: none)."""
    return int(_lib.load().kda_fwd_workspace_bytes(n_seqs, n_tokens, H, d_k, d_v, _dt(dtype)))


def kda_fwd_chunked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, S0: Optional[torch.Tensor] = None,
                    cu_seqlens: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None,
                    output_final_state: bool = True,
                    o: Optional[torch.Tensor] = None,
                    S_T: Optional[torch.Tensor] = None,
                    workspace: Union[None, bool, torch.Tensor] = None,
                    ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked KDA prefill.

    q, k : [B, T, H, d_k] or packed [N, H, d_k] (bf16 or fp32); v : [..., H, d_v]
    g    : [..., H, d_k] fp32 log-decay in [-5, 0];  beta : [..., H] fp32
    S0   : [n_seqs, H, d_k, d_v] fp32 or None
    cu_seqlens : int32 [n_seqs + 1] on the device (packed input only)
    workspace  : None or True -> a torch buffer of kda_fwd_workspace_bytes is
                 allocated here when that size is nonzero (the library itself
                 allocates nothing); False -> no workspace (single pass);
                 a contiguous uint8 device tensor -> used as given
    Returns (o [same leading shape, d_v], S_T [n_seqs, H, d_k, d_v] or None).
    """
    dev = q.device
    if q.dim() == 4:
        if cu_seqlens is not None and q.shape[0] != 1:
            raise ValueError("cu_seqlens needs packed input ([N, H, d] or [1, N, H, d])")
        lead = tuple(q.shape[:2])
        n_seqs = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
        N = q.shape[0] * q.shape[1]
        H, dk = q.shape[2], q.shape[3]
    elif q.dim() == 3:
        lead = (q.shape[0],)
        N, H, dk = q.shape
        if cu_seqlens is None:
            n_seqs = 1
        else:
            n_seqs = cu_seqlens.numel() - 1
    else:
        raise ValueError("q must be [B, T, H, d_k] or [N, H, d_k]")
    dv = v.shape[-1]
    _need(q, "q", device=dev)
    _need(k, "k", dtype=q.dtype, shape=q.shape, device=dev)
    _need(v, "v", dtype=q.dtype, shape=lead + (H, dv), device=dev)
    _need(g, "g", dtype=torch.float32, shape=lead + (H, dk), device=dev)
    _need(beta, "beta", dtype=torch.float32, shape=lead + (H,), device=dev)
    if S0 is not None:
        _need(S0, "S0", dtype=torch.float32, shape=(n_seqs, H, dk, dv), device=dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, device=dev)
    in_dt = _dt(q.dtype)
    od = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty(lead + (H, dv), dtype=od, device=dev)
    else:
        _need(o, "o", dtype=od, shape=lead + (H, dv), device=dev)
    if output_final_state and S_T is None:
        S_T = torch.empty((n_seqs, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _need(S_T, "S_T", dtype=torch.float32, shape=(n_seqs, H, dk, dv), device=dev)
    lib = _lib.load()
    ws, ws_bytes = None, 0
    if isinstance(workspace, torch.Tensor):
        _need(workspace, "workspace", dtype=torch.uint8, device=dev)
        ws, ws_bytes = workspace, workspace.numel()
    elif workspace is None or workspace is True:
        need = 0 if (cu_seqlens is not None and n_seqs > 1) else \
            int(lib.kda_fwd_workspace_bytes(n_seqs, N, H, dk, dv, in_dt))
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            ws_bytes = need
    st = lib.kda_fwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                             _ptr(cu_seqlens), n_seqs, N, H, dk, dv, in_dt, _dt(od),
                             _ptr(o), _ptr(S_T), _ptr(ws), ws_bytes, _stream(dev))
    _lib.check(st)
    return o, S_T


def kda_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, S: torch.Tensor,
                    out_dtype: Optional[torch.dtype] = None,
                    o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode token per sequence.  q, k, g : [N, H, d_k]; v : [N, H, d_v];
    beta : [N, H]; S : [N, H, d_k, d_v] fp32, updated in place.  Returns o."""
    dev = q.device
    if q.dim() != 3:
        raise ValueError("q must be [N, H, d_k]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q", device=dev)
    _need(k, "k", dtype=q.dtype, shape=q.shape, device=dev)
    _need(v, "v", dtype=q.dtype, shape=(N, H, dv), device=dev)
    _need(g, "g", dtype=torch.float32, shape=(N, H, dk), device=dev)
    _need(beta, "beta", dtype=torch.float32, shape=(N, H), device=dev)
    _need(S, "S", dtype=torch.float32, shape=(N, H, dk, dv), device=dev)
    od = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, H, dv), dtype=od, device=dev)
    else:
        _need(o, "o", dtype=od, shape=(N, H, dv), device=dev)
    lib = _lib.load()
    st = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S),
                             N, H, dk, dv, _dt(q.dtype), _dt(od), _ptr(o), _stream(dev))
    _lib.check(st)
    return o


def _draft_shapes(q, k, v, g, beta, name="q"):
    if q.dim() != 4:
        raise ValueError(f"{name} must be [N, K, H, d_k]")
    N, K, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(q, name, device=dev)
    _need(k, "k", dtype=q.dtype, shape=q.shape, device=dev)
    _need(v, "v", dtype=q.dtype, shape=(N, K, H, dv), device=dev)
    _need(g, "g", dtype=torch.float32, shape=(N, K, H, dk), device=dev)
    _need(beta, "beta", dtype=torch.float32, shape=(N, K, H), device=dev)
    return N, K, H, dk, dv


def kda_decode_verify(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                      beta: torch.Tensor, S: torch.Tensor,
                      out_dtype: Optional[torch.dtype] = None,
                      o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Outputs of K drafted tokens per sequence without committing them.
    q, k, g : [N, K, H, d_k]; v : [N, K, H, d_v]; beta : [N, K, H];
    S : [N, H, d_k, d_v] fp32, read only.  Returns o [N, K, H, d_v]."""
    N, K, H, dk, dv = _draft_shapes(q, k, v, g, beta)
    dev = q.device
    _need(S, "S", dtype=torch.float32, shape=(N, H, dk, dv), device=dev)
    od = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, K, H, dv), dtype=od, device=dev)
    else:
        _need(o, "o", dtype=od, shape=(N, K, H, dv), device=dev)
    st = _lib.load().kda_decode_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S),
                                       N, K, H, dk, dv, _dt(q.dtype), _dt(od), _ptr(o),
                                       _stream(dev))
    _lib.check(st)
    return o


def kda_decode_commit(k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                      n_accept: torch.Tensor, S: torch.Tensor) -> None:
    """Replay the first n_accept[n] of the K cached tokens of sequence n into
    S (in place).  k, g : [N, K, H, d_k]; v : [N, K, H, d_v]; beta :
    [N, K, H]; n_accept : int32 [N] on the device."""
    N, K, H, dk, dv = _draft_shapes(k, k, v, g, beta, name="k")
    dev = k.device
    _need(S, "S", dtype=torch.float32, shape=(N, H, dk, dv), device=dev)
    _need(n_accept, "n_accept", dtype=torch.int32, shape=(N,), device=dev)
    st = _lib.load().kda_decode_commit(_ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(n_accept),
                                       _ptr(S), N, K, H, dk, dv, _dt(k.dtype), _stream(dev))
    _lib.check(st)


def kda_decode_spec(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, S: torch.Tensor, prev: Optional[dict] = None,
                    n_accept: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None,
                    o: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One speculative decode step: commit prev's accepted drafts (a dict of
    k, v, g, beta shaped [N, K_prev, H, ...], n_accept int32 [N]) into S,
    then verify the new drafts q, k, v, g, beta [N, K, H, ...] from it.
    Returns o [N, K, H, d_v]; S is updated in place."""
    N, K, H, dk, dv = _draft_shapes(q, k, v, g, beta)
    dev = q.device
    _need(S, "S", dtype=torch.float32, shape=(N, H, dk, dv), device=dev)
    Kp = 0
    pk = pv = pg = pb = None
    if prev is not None:
        pk, pv, pg, pb = prev["k"], prev["v"], prev["g"], prev["beta"]
        Np, Kp, Hp, dkp, dvp = _draft_shapes(pk, pk, pv, pg, pb, name="prev k")
        if (Np, Hp, dkp, dvp) != (N, H, dk, dv) or pk.dtype != q.dtype:
            raise ValueError("prev drafts must match the new drafts in N, H, d and dtype")
        if n_accept is None:
            raise ValueError("n_accept is required with prev")
        _need(n_accept, "n_accept", dtype=torch.int32, shape=(N,), device=dev)
    od = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, K, H, dv), dtype=od, device=dev)
    else:
        _need(o, "o", dtype=od, shape=(N, K, H, dv), device=dev)
    st = _lib.load().kda_decode_spec(_ptr(pk), _ptr(pv), _ptr(pg), _ptr(pb),
                                     _ptr(n_accept) if prev is not None else None, Kp,
                                     _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), K, _ptr(S),
                                     N, H, dk, dv, _dt(q.dtype), _dt(od), _ptr(o), _stream(dev))
    _lib.check(st)
    return o


def kda_fwd_chunked_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, z: torch.Tensor,
                          A_log: torch.Tensor, b: torch.Tensor,
                          S0: Optional[torch.Tensor] = None,
                          cu_seqlens: Optional[torch.Tensor] = None,
                          out_dtype: Optional[torch.dtype] = None,
                          output_final_state: bool = True,
                          o: Optional[torch.Tensor] = None,
                          S_T: Optional[torch.Tensor] = None,
                          workspace: Union[None, bool, torch.Tensor] = None,
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill with the gate and q/k preprocessing fused in:
    q, k unnormalised [..., H, d_k]; z [..., H, d_k] (gate pre-activation,
    q's dtype); A_log [H] fp32; b [..., H] (beta pre-activation, q's dtype).
    g = -5 sigmoid(exp(A_log) z), beta = sigmoid(b), q and k L2-normalised
    in the kernel.  Other arguments as kda_fwd_chunked."""
    dev = q.device
    if q.dim() == 4:
        if cu_seqlens is not None and q.shape[0] != 1:
            raise ValueError("cu_seqlens needs packed input ([N, H, d] or [1, N, H, d])")
        lead = tuple(q.shape[:2])
        n_seqs = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
        N, H, dk = q.shape[0] * q.shape[1], q.shape[2], q.shape[3]
    elif q.dim() == 3:
        lead = (q.shape[0],)
        N, H, dk = q.shape
        n_seqs = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    else:
        raise ValueError("q must be [B, T, H, d_k] or [N, H, d_k]")
    dv = v.shape[-1]
    _need(q, "q", device=dev)
    _need(k, "k", dtype=q.dtype, shape=q.shape, device=dev)
    _need(v, "v", dtype=q.dtype, shape=lead + (H, dv), device=dev)
    _need(z, "z", dtype=q.dtype, shape=q.shape, device=dev)
    _need(b, "b", dtype=q.dtype, shape=lead + (H,), device=dev)
    _need(A_log, "A_log", dtype=torch.float32, shape=(H,), device=dev)
    if S0 is not None:
        _need(S0, "S0", dtype=torch.float32, shape=(n_seqs, H, dk, dv), device=dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, device=dev)
    in_dt = _dt(q.dtype)
    od = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty(lead + (H, dv), dtype=od, device=dev)
    else:
        _need(o, "o", dtype=od, shape=lead + (H, dv), device=dev)
    if output_final_state and S_T is None:
        S_T = torch.empty((n_seqs, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _need(S_T, "S_T", dtype=torch.float32, shape=(n_seqs, H, dk, dv), device=dev)
    lib = _lib.load()
    ws, ws_bytes = None, 0
    if isinstance(workspace, torch.Tensor):
        _need(workspace, "workspace", dtype=torch.uint8, device=dev)
        ws, ws_bytes = workspace, workspace.numel()
    elif workspace is None or workspace is True:
        need = 0 if (cu_seqlens is not None and n_seqs > 1) else \
            int(lib.kda_fwd_workspace_bytes(n_seqs, N, H, dk, dv, in_dt))
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            ws_bytes = need
    st = lib.kda_fwd_chunked_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A_log), _ptr(b),
                                   _ptr(S0), _ptr(cu_seqlens), n_seqs, N, H, dk, dv, in_dt,
                                   _dt(od), _ptr(o), _ptr(S_T), _ptr(ws), ws_bytes,
                                   _stream(dev))
    _lib.check(st)
    return o, S_T


def kda_bwd_workspace_bytes(n_seqs: int, n_tokens: int, H: int, d_k: int, d_v: int) -> int:
    """Bytes of workspace kda_bwd_chunked needs for these sizes."""
    return int(_lib.load().kda_bwd_workspace_bytes(n_seqs, n_tokens, H, d_k, d_v))


def kda_bwd_chunked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, dO: torch.Tensor, S0: Optional[torch.Tensor] = None,
                    dS_T: Optional[torch.Tensor] = None,
                    cu_seqlens: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, ...]:
    """Gradients of kda_fwd_chunked: (dq, dk, dv, dg, dbeta, dS0), fp32, the
    inputs' shapes; dO has o's shape and q's dtype, dS_T the final state's
    (or None).  The workspace (uint8) is allocated through torch unless
    given."""
    dev = q.device
    if q.dim() == 4:
        if cu_seqlens is not None and q.shape[0] != 1:
            raise ValueError("cu_seqlens needs packed input ([N, H, d] or [1, N, H, d])")
        lead = tuple(q.shape[:2])
        n_seqs = q.shape[0] if cu_seqlens is None else cu_seqlens.numel() - 1
        N, H, dk = q.shape[0] * q.shape[1], q.shape[2], q.shape[3]
    elif q.dim() == 3:
        lead = (q.shape[0],)
        N, H, dk = q.shape
        n_seqs = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    else:
        raise ValueError("q must be [B, T, H, d_k] or [N, H, d_k]")
    dv = v.shape[-1]
    _need(q, "q", device=dev)
    _need(k, "k", dtype=q.dtype, shape=q.shape, device=dev)
    _need(v, "v", dtype=q.dtype, shape=lead + (H, dv), device=dev)
    _need(g, "g", dtype=torch.float32, shape=lead + (H, dk), device=dev)
    _need(beta, "beta", dtype=torch.float32, shape=lead + (H,), device=dev)
    _need(dO, "dO", dtype=q.dtype, shape=lead + (H, dv), device=dev)
    st_shape = (n_seqs, H, dk, dv)
    if S0 is not None:
        _need(S0, "S0", dtype=torch.float32, shape=st_shape, device=dev)
    if dS_T is not None:
        _need(dS_T, "dS_T", dtype=torch.float32, shape=st_shape, device=dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, device=dev)
    lib = _lib.load()
    need = kda_bwd_workspace_bytes(n_seqs, N, H, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", dtype=torch.uint8, device=dev)
    f32 = lambda shape: torch.empty(shape, dtype=torch.float32, device=dev)   # noqa: E731
    dq, dkk, dg = f32(lead + (H, dk)), f32(lead + (H, dk)), f32(lead + (H, dk))
    dvv, db, dS0 = f32(lead + (H, dv)), f32(lead + (H,)), f32(st_shape)
    st = lib.kda_bwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                             _ptr(cu_seqlens), n_seqs, N, H, dk, dv, _dt(q.dtype), _ptr(dO),
                             _ptr(dS_T), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg), _ptr(db),
                             _ptr(dS0), _ptr(workspace), workspace.numel(), _stream(dev))
    _lib.check(st)
    return dq, dkk, dvv, dg, db, dS0
