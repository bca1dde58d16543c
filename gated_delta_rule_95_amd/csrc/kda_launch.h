// Internal launch interface between the C-ABI layer (kda_api.cpp) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

struct DecodeArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    float *S;
    void *o;
    int32_t N, H, d_k, d_v;
    bool in_bf16, out_bf16;
    void *stream;
};

struct PrefillArgs {
    const void *q, *k, *v;
    const float *g, *beta, *S0;
    const int32_t *cu_seqlens;   // nullptr: equal lengths seqlen
    int32_t n_seqs;
    int64_t n_tokens;
    int32_t seqlen;              // used when cu_seqlens == nullptr
    int32_t H, d_k, d_v;
    bool in_bf16, out_bf16;
    void *o;
    float *S_T;
    void *workspace;             // caller scratch (nullptr: single pass)
    size_t workspace_bytes;
    // gated prologue (kda_fwd_chunked_gated): z and b in the input type
    // replace g and beta; A_log [H]; q and k arrive unnormalised
    bool gated;
    const void *z, *b;
    const float *A_log;
    // non-null: the checkpointing forward of the backward pass (single pass,
    // not gated, o not written): the state at every chunk start goes to
    // slot bos / 16 + n + c, in 16 x 16 tiles (layout at the prefill kernel)
    float *ckpt;
    void *stream;
};

// Speculative decoding (kda_decode_verify / _commit / _spec): replay up to
// Kr cached tokens per sequence (n_accept[n] of them) into S, optionally
// write S, then run K drafts from the result and write their outputs.
constexpr int kSpecMaxTokens = 16;
struct SpecArgs {
    const void *rk, *rv;             // [N, Kr, H, d] replayed tokens
    const float *rg, *rbeta;
    const int32_t *n_accept;         // [N] or nullptr (nothing replayed)
    int32_t Kr;
    const void *q, *k, *v;           // [N, K, H, d] drafts
    const float *g, *beta;
    void *o;                         // [N, K, H, d_v]
    int32_t K;
    float *S;
    int32_t N, H, d_k, d_v;
    bool in_bf16, out_bf16, write_state;
    void *stream;
};

// Chunked backward (kda_bwd_chunked): the sweep over column blocks and the
// per-chunk finisher; ckpt holds the forward's chunk-start states, part the
// blocks' partial sums, both indexed by chunk slot bos / 16 + n + c.
struct BwdArgs {
    const void *q, *k, *v, *dO;
    const float *g, *beta, *dST;
    const int32_t *cu_seqlens;
    int32_t n_seqs;
    int64_t n_tokens;
    int32_t seqlen, H, d_k, d_v;
    bool in_bf16;
    float *ckpt, *part;
    int64_t n_slots;
    float *dq, *dk, *dv, *dg, *dbeta, *dS0;
    void *stream;
};
// floats of partial sums per (chunk slot, head)
size_t bwd_part_floats(int32_t d_k, int32_t d_v);

hipError_t launch_decode(const DecodeArgs &a);
hipError_t launch_spec(const SpecArgs &a);
hipError_t launch_bwd(const BwdArgs &a);
// Bytes of workspace the sequence-split path needs for these sizes on the
// current device (0: the single-pass kernel is used).  Reads only the size
// fields of `a` (and whether cu_seqlens is set).
size_t prefill_workspace_bytes(const PrefillArgs &a);
hipError_t launch_prefill(const PrefillArgs &a);

// Records a message for kda_last_error() on the calling thread and returns s.
kda_status set_error(kda_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace kda
