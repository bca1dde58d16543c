/*
 * libkda -- Kimi Delta Attention (KDA) on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes; no C++ or framework types cross it.
 *
 * What is computed.  Per head, KDA keeps a d_k x d_v state S whose rows are
 * key channels and, for every token t, applies
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                               alpha_t = exp(g_t)
 *
 * (Kimi K3 architecture walkthrough, mhpq.cn/news/56770, section
 * "KDA 到底在算什么": the state-update equation and, in its figure caption,
 * the order decay -> erase along k_t -> write; the read uses the updated
 * state.  alpha = exp(g) with g bounded below by -5: K3-on-TPU essay,
 * blog.higcp.com, section "KDA + Gated MLA", lower-bounded decay.)
 * No attention scale is applied to q.
 *
 * Layouts (all dense, row-major, token-major, no padding):
 *     q, k    [n_tokens, H, d_k]      dtype = in_dtype
 *     v       [n_tokens, H, d_v]      dtype = in_dtype
 *     o       [n_tokens, H, d_v]      dtype = out_dtype
 *     g       [n_tokens, H, d_k]      float32, natural-log decay, g in [-5, 0]
 *     beta    [n_tokens, H]           float32, beta in [0, 1]
 *     S0, S_T, S  [n_seqs, H, d_k, d_v]  float32, row = key channel
 *     cu_seqlens  int32 [n_seqs + 1], cu_seqlens[0] = 0, non-decreasing,
 *                 cu_seqlens[n_seqs] = n_tokens (device memory)
 * The packed (varlen) layout follows the pages' description of a KDA
 * implementation that packs variable-length sequences and keeps one
 * recurrent state per sequence (K3-on-TPU essay, "KDA + Gated MLA" and the
 * section on the existing TPU kernel).
 *
 * Alignment (bytes; the widest vector access the kernels make): q, k: two
 * elements; v, o: four elements; g: 8 (prefill) / 4 (decode); beta, S0,
 * S_T: 4; the decode state S: 16.  Any slice of a contiguous tensor along
 * its token (or sequence) axis satisfies these.
 *
 * Ownership: the caller allocates every buffer in device memory (any HIP
 * allocator) and keeps it alive until the work queued on `stream` is done.
 * The library allocates no device memory, keeps no pointer after a call
 * returns, and never synchronises the host.
 *
 * Errors: every entry point returns a kda_status; nothing aborts or throws
 * across the ABI.  Argument problems are found on the host before anything
 * is launched (nothing is written then).  A launch failure returns
 * KDA_ERR_HIP.  kda_last_error() gives a message for the calling thread's
 * most recent failure.  Values inside device buffers (cu_seqlens order, the
 * range of g and beta) are preconditions that are NOT checked: g < -5 can
 * overflow the bf16 rescale factors (the 16-token tile bound of the pages
 * assumes g >= -5) and is undefined behaviour.  The prefill clamps every
 * cu_seqlens entry into [0, n_tokens] before use, so a cu_seqlens that
 * breaks its contract (decreasing, negative, or beyond n_tokens) yields
 * unspecified o and S_T but never an access outside the buffers.
 *
 * Concurrency: calls are asynchronous on `stream` and re-entrant.  Calls
 * that write the same buffers must be ordered by the caller.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_VERSION_MAJOR 0
#define KDA_VERSION_MINOR 1

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer  */
    KDA_ERR_UNSUPPORTED = 2, /* head size or dtype combination not built    */
    KDA_ERR_HIP = 3          /* the HIP runtime reported an error           */
} kda_status;

typedef enum kda_dtype {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype;

/* Opaque stream handle: a hipStream_t (0 = the default stream). */
typedef void *kda_stream_t;

/*
 * kda_fwd_chunked -- chunked prefill over a packed batch of sequences.
 *
 * For every sequence n (tokens cu_seqlens[n] .. cu_seqlens[n+1]-1) and head
 * h, runs the recurrence above from S0[n, h] (zeros when S0 == NULL), writes
 * o for every token and the final state to S_T[n, h] (skipped when
 * S_T == NULL).  An empty sequence gives S_T[n] = S0[n] (or zeros).
 * When cu_seqlens == NULL the batch is n_seqs sequences of equal length
 * n_tokens / n_seqs laid out back to back ([B, T, H, d] == [B*T, H, d]);
 * n_tokens must then be a multiple of n_seqs.
 *
 * The work is split into 16-token chunks (the decay tile of the pages: with
 * g >= -5 a tile's cumulative log-decay stays in (-80, 0), so its rescale
 * factors e^{+-80} fit bf16 and fp32).  Inside a chunk the WY/UT form
 * (I + A)^{-1} Diag(beta) with A = strict_lower(Diag(beta) K~ K^T) is used;
 * bf16 inputs run on bf16 matrix cores with fp32 accumulation (intra-chunk
 * operands as bf16 hi/lo pairs), fp32 inputs on fp32 matrix cores.  The
 * state is carried in fp32 between chunks.
 *
 * Arguments
 *   q, k, v, g, beta   inputs, layouts above
 *   S0                 float32 entry states or NULL
 *   cu_seqlens         int32 device array or NULL (equal lengths)
 *   n_seqs             number of sequences, >= 0 (0: nothing is done)
 *   n_tokens           total tokens, 0 <= n_tokens <= 2^31 - 64
 *   H                  heads, >= 1, with H * max(d_k, d_v) < 2^25
 *   d_k, d_v           16, 32, 64 or 128 each
 *   in_dtype           KDA_BF16 or KDA_F32 (q, k, v)
 *   out_dtype          dtype of o: KDA_BF16 (bf16 inputs only) or KDA_F32;
 *                      fp32 o is exact fp32 accumulation before any rounding
 *   o                  output (may be NULL iff n_tokens == 0)
 *   S_T                float32 final states or NULL
 *   workspace          caller-owned device scratch, or NULL
 *   workspace_bytes    its size; see kda_fwd_workspace_bytes
 *   stream             hipStream_t
 *
 * Workspace.  With workspace == NULL and workspace_bytes == 0 the call runs
 * the single-pass kernel, which needs no scratch.  With a workspace of at
 * least kda_fwd_workspace_bytes(n_seqs, n_tokens, H, d_k, d_v, in_dtype)
 * bytes (256-byte aligned) the library may instead split long sequences
 * into segments processed side by side on the device (sequence-split path,
 * below), which is worthwhile when sequences x heads are too few to fill the
 * GPU.  A non-NULL workspace that is smaller than that, or misaligned, is
 * rejected with KDA_ERR_INVALID_ARG.  The contents of the workspace are
 * undefined after the call; it may not overlap any other argument, and two
 * calls that are in flight at the same time need separate workspaces.
 *
 * Sequence-split path.  Each long sequence is cut into segments.  The first
 * runs from S0 as usual; every later segment runs from a zero state and, in
 * the same launch, also carries the d_k columns of its transition matrix
 * M (the product of its tokens' maps S -> (I - b k k^T) Diag(alpha) S),
 * which gives the segment's affine summary S_end = M S_entry + S~ and, per
 * token, the query pulled back to the segment start, R_t = Phi_t^T q_t.  A
 * scan over segments then gives every segment's true entry state, and a
 * correction adds R_t S_entry to the zero-start outputs.  This is the
 * affine-summary-and-prefix-scan scheme the K3-on-TPU essay describes for
 * context parallelism over KDA (blog.higcp.com, the section on the existing
 * TPU kernel), used here across compute units of one GPU, which the same
 * essay names as KDA's intra-device sequence-parallel regime ("KDA + Gated
 * MLA", the costs section, item (3)).  Results agree with the single-pass
 * path to rounding.
 */
kda_status kda_fwd_chunked(const void *q, const void *k, const void *v,
                           const float *g, const float *beta, const float *S0,
                           const int32_t *cu_seqlens, int32_t n_seqs,
                           int64_t n_tokens, int32_t H, int32_t d_k, int32_t d_v,
                           kda_dtype in_dtype, kda_dtype out_dtype, void *o,
                           float *S_T, void *workspace, size_t workspace_bytes,
                           kda_stream_t stream);

/*
 * kda_fwd_chunked_gated -- kda_fwd_chunked with the gate and q/k
 * preprocessing fused into its loads.
 *
 * Instead of g, beta and normalised q, k it takes what the model's
 * projections produce and forms, per token and head:
 *     q <- q / sqrt(|q|^2 + 1e-6),  k <- k / sqrt(|k|^2 + 1e-6)
 *     g = -5 sigmoid(exp(A_log[h]) z)   (per key channel)
 *     beta = sigmoid(b)
 * The gate is K3's lower-bounded parameterisation (K3-on-TPU essay,
 * blog.higcp.com, "KDA + Gated MLA", lower-bounded decay: g_min = -5, A a
 * per-head log-scale); q/k L2 normalisation and the sigmoid branches giving
 * the per-channel gate and the scalar beta are the Q/K preprocessing the K3
 * architecture walkthrough describes (mhpq.cn/news/56770, after "KDA 到底在
 * 算什么").  The epsilon of the normalisation is not given by the pages.
 * The short causal convolution and Swish that precede the normalisation there
 * are not included.  Compared with kda_fwd_chunked this reads z in the
 * input type instead of an fp32 g, and b instead of an fp32 beta.
 *
 *   q, k   [n_tokens, H, d_k] in_dtype, unnormalised
 *   z      [n_tokens, H, d_k] in_dtype, gate pre-activation
 *   A_log  [H] float32
 *   b      [n_tokens, H] in_dtype, beta pre-activation
 * Every other argument, the workspace and the errors are those of
 * kda_fwd_chunked (kda_fwd_workspace_bytes applies unchanged).  Alignment:
 * z as q, b one element.
 */
kda_status kda_fwd_chunked_gated(const void *q, const void *k, const void *v, const void *z,
                                 const float *A_log, const void *b, const float *S0,
                                 const int32_t *cu_seqlens, int32_t n_seqs, int64_t n_tokens,
                                 int32_t H, int32_t d_k, int32_t d_v, kda_dtype in_dtype,
                                 kda_dtype out_dtype, void *o, float *S_T, void *workspace,
                                 size_t workspace_bytes, kda_stream_t stream);

/*
 * kda_fwd_workspace_bytes -- scratch size for kda_fwd_chunked.
 *
 * Returns the number of bytes of workspace with which kda_fwd_chunked, called
 * with the same sizes on the current device, may take the sequence-split
 * path; 0 when it would not split (then no workspace is used).  The size
 * holds the segments' affine summaries and per-token pull-back operands, so
 * it grows with the number of tokens (at most with the number of chunks)
 * and never with the state of a longer sequence (the state size does not
 * depend on T).  For n_seqs > 1 it assumes equal lengths (cu_seqlens ==
 * NULL); a packed batch of several sequences never uses the workspace.
 * Invalid sizes give 0 (kda_fwd_chunked then reports the error).
 */
size_t kda_fwd_workspace_bytes(int32_t n_seqs, int64_t n_tokens, int32_t H, int32_t d_k,
                               int32_t d_v, kda_dtype in_dtype);

/*
 * kda_fwd_chunked_noalloc -- kda_fwd_chunked for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, layouts, results and errors as kda_fwd_chunked, without
 * the workspace pair: where kda_fwd_chunked would use a workspace (the
 * sequence-split path, kda_fwd_workspace_bytes > 0) this call takes it from
 * a fixed array of KDA_NOALLOC_SCRATCH_BYTES that the library holds on each
 * device it runs on, until the process ends; nothing is allocated or freed.
 * Sizes whose workspace exceeds that are rejected with KDA_ERR_INVALID_ARG
 * (kda_fwd_chunked with a caller workspace serves them).  Every call on a
 * device shares that device's array and leaves its contents behind (every
 * element the split path reads is written earlier in the same call, so
 * nothing needs clearing): calls that overlap in time on one device, on
 * different streams or threads, race and must be ordered by the caller.
 * The array's address on a device is looked up at that device's first call.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_fwd_chunked_noalloc(const void *q, const void *k, const void *v,
                                   const float *g, const float *beta, const float *S0,
                                   const int32_t *cu_seqlens, int32_t n_seqs,
                                   int64_t n_tokens, int32_t H, int32_t d_k, int32_t d_v,
                                   kda_dtype in_dtype, kda_dtype out_dtype, void *o,
                                   float *S_T, kda_stream_t stream);

/*
 * kda_decode_step -- one new token for each of N independent sequences.
 *
 * Applies the recurrence once per (sequence n, head h), updating
 * S[n, h] (float32, [N, H, d_k, d_v]) IN PLACE, and writes o[n, h].  The
 * in-place update is how the pages describe KDA decoding (K3-on-TPU essay,
 * "KDA + Gated MLA", the costs section on speculative decoding).  The state
 * is read once and written once; the step is bound by HBM bandwidth
 * (the AI-accelerator checklist, lishengnan.com/aichip, "Decode: bandwidth
 * roof first").
 *
 * Arguments
 *   q, k      [N, H, d_k] in_dtype;  v [N, H, d_v] in_dtype
 *   g         [N, H, d_k] float32;   beta [N, H] float32
 *   S         [N, H, d_k, d_v] float32, read and overwritten
 *   N, H      >= 0, >= 1;  d_k, d_v in {16, 32, 64, 128}
 *   o         [N, H, d_v] out_dtype
 * S must not overlap any other argument, nor o an input.
 */
kda_status kda_decode_step(const void *q, const void *k, const void *v,
                           const float *g, const float *beta, float *S,
                           int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                           kda_dtype in_dtype, kda_dtype out_dtype, void *o,
                           kda_stream_t stream);

/*
 * Speculative decoding: verify drafted tokens, replay the accepted ones.
 *
 * The decode step updates the state in place, so once a draft is rejected
 * the state cannot be rolled back, and keeping a state snapshot per draft
 * position multiplies the state traffic that dominates large-batch serving.
 * The pages describe K3 keeping only each draft's inputs and replaying the
 * accepted ones on chip to rebuild the state (K3-on-TPU essay,
 * blog.higcp.com, "KDA + Gated MLA", the costs section, item (1)).  These
 * calls do that for the KDA recurrence; the drafts' inputs are the caller's
 * (the cache of "projected inputs").
 *
 * Token tensors hold K tokens per sequence, token-major within a sequence:
 *     q, k, g  [N, K, H, d_k]    v, o  [N, K, H, d_v]    beta  [N, K, H]
 * (dtypes as for kda_decode_step); S is [N, H, d_k, d_v] float32; n_accept
 * is int32 [N] in device memory, each entry clamped into [0, K] (an entry
 * out of range changes the result, never the addresses touched).
 * 1 <= K <= 16 for drafts (0 <= K <= 16 for kda_decode_commit).  Alignment
 * as for kda_decode_step.  Errors as for the other entry points.
 *
 * kda_decode_verify  runs the K drafts of every sequence from S and writes
 *     o for each draft position (o[n, j] is what decoding drafts 0..j one at
 *     a time would output).  S is read only.
 * kda_decode_commit  replays the first n_accept[n] tokens of sequence n
 *     into S[n] (in place), as that many kda_decode_step calls would.
 * kda_decode_spec    one pass of both, for a decode loop: first commits the
 *     previous step's drafts (k_prev ... beta_prev, K_prev per sequence,
 *     n_accept[n] of them accepted; K_prev = 0 and NULL pointers for none)
 *     into S, then verifies the K new drafts from the updated S.  The state
 *     is read once and written once, the traffic of one decode step.
 */
kda_status kda_decode_verify(const void *q, const void *k, const void *v, const float *g,
                             const float *beta, const float *S, int32_t N, int32_t K,
                             int32_t H, int32_t d_k, int32_t d_v, kda_dtype in_dtype,
                             kda_dtype out_dtype, void *o, kda_stream_t stream);
kda_status kda_decode_commit(const void *k, const void *v, const float *g, const float *beta,
                             const int32_t *n_accept, float *S, int32_t N, int32_t K,
                             int32_t H, int32_t d_k, int32_t d_v, kda_dtype in_dtype,
                             kda_stream_t stream);
kda_status kda_decode_spec(const void *k_prev, const void *v_prev, const float *g_prev,
                           const float *beta_prev, const int32_t *n_accept, int32_t K_prev,
                           const void *q, const void *k, const void *v, const float *g,
                           const float *beta, int32_t K, float *S, int32_t N, int32_t H,
                           int32_t d_k, int32_t d_v, kda_dtype in_dtype, kda_dtype out_dtype,
                           void *o, kda_stream_t stream);

/*
 * kda_bwd_chunked -- gradients of kda_fwd_chunked.
 *
 * Given the forward's inputs and the cotangents dO of o ([n_tokens, H, d_v],
 * in_dtype) and dS_T of the final states (float32 [n_seqs, H, d_k, d_v], or
 * NULL for zero), writes float32 gradients with the inputs' layouts:
 * dq, dk, dg [n_tokens, H, d_k]; dv [n_tokens, H, d_v]; dbeta [n_tokens, H];
 * dS0 [n_seqs, H, d_k, d_v] (skipped when NULL).  A backward pass (custom
 * VJP) is one of the parts of the KDA kernel suite the K3-on-TPU essay
 * describes (blog.higcp.com, the section on the existing TPU kernel).
 *
 * It reruns the forward keeping the state at every 16-token chunk start,
 * then walks the chunks backwards carrying the cotangent of the state, by
 * blocks of state columns (writing dv and dS0), and forms each chunk's dq,
 * dk, dg and dbeta in a second, chunk-parallel pass.  bf16 inputs with
 * d_k >= 32 run on the matrix cores (bf16 hi/lo operand pairs, fp32
 * accumulation); fp32 inputs and d_k = 16 run in fp32 on the vector ALU.
 * The workspace (required) must hold kda_bwd_workspace_bytes(...) bytes,
 * 256-byte aligned: the state checkpoints (64 KiB per chunk and head at
 * d = 128) and as much again for the chunk-exit cotangents (or the column
 * blocks' partial sums).  Pointers must be aligned to the widest access
 * made on them: q, k to 2 elements, v, dO to 4 elements, g to 8 bytes, dq
 * and dk to 16 bytes, the rest to 4 bytes.  Other arguments, layouts and
 * errors as for kda_fwd_chunked.
 */
size_t kda_bwd_workspace_bytes(int32_t n_seqs, int64_t n_tokens, int32_t H, int32_t d_k,
                               int32_t d_v);
kda_status kda_bwd_chunked(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *S0, const int32_t *cu_seqlens,
                           int32_t n_seqs, int64_t n_tokens, int32_t H, int32_t d_k,
                           int32_t d_v, kda_dtype in_dtype, const void *dO, const float *dS_T,
                           float *dq, float *dk, float *dv, float *dg, float *dbeta, float *dS0,
                           void *workspace, size_t workspace_bytes, kda_stream_t stream);

/* Human-readable name of a status code (static string). */
const char *kda_status_string(kda_status s);

/* Message for the calling thread's most recent failing call ("" if none). */
const char *kda_last_error(void);

/* "major.minor" plus the offload target the library was built for. */
const char *kda_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
