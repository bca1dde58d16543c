"""Seeded synthetic inputs for the KDA (Kimi Delta Attention) workloads.

This module is shared by the CPU oracle and the HIP path; it holds none of
the recurrence's arithmetic.  It only draws random tensors with the shapes
and value distributions of the workloads, rounds them to bfloat16 where the
workload asks for bf16, and lays them out token-major:

    q, k, g : [tokens, H, d_k]     v : [tokens, H, d_v]
    beta    : [tokens, H]          S0 / S : [n_seqs, H, d_k, d_v]
    cu_seqlens : int32 [n_seqs + 1]

Every (sequence, head, tensor) triple has its own counter-free PCG64 stream
keyed by ``SeedSequence(base_seed, spawn_key=(seq, head, tensor_id))``, so one
head of one sequence can be regenerated on the host (for the oracle) without
materialising the whole batch.

The L2 normalisation of q/k and the sigmoid in the gate distribution are part
of how the inputs are *drawn* (the kernel's callers hand it already-normalised
keys and already-bounded log-decays); they are not steps of the method.
"""
from __future__ import annotations

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits,
    bf16_bits_to_f32,
    round_bf16,
    head_inputs,
    decode_head_inputs,
    batch_inputs,
    decode_batch_inputs,
    draft_batch_inputs,
    seq_lengths,
    cu_seqlens,
)
