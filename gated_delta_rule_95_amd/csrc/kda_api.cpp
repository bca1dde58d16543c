// C-ABI layer of libkda: argument validation, dtype/shape dispatch, errors.
// Declarations and the contract of every entry point are in include/kda.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kda.h"
#include "kda_launch.h"

#define KDA_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

kda_status fail(kda_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

kda_status ok()
{
    g_err[0] = '\0';
    return KDA_OK;
}

bool head_dim_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

kda_status check_dtypes(kda_dtype in, kda_dtype out)
{
    if (in != KDA_F32 && in != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARG, "in_dtype %d is not a kda_dtype", (int)in);
    if (out != KDA_F32 && out != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARG, "out_dtype %d is not a kda_dtype", (int)out);
    if (in == KDA_F32 && out == KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "fp32 inputs with a bf16 output are not supported");
    return KDA_OK;
}

kda_status check_dims(int32_t H, int32_t d_k, int32_t d_v)
{
    if (H < 1) return fail(KDA_ERR_INVALID_ARG, "H must be >= 1 (got %d)", H);
    if (!head_dim_ok(d_k) || !head_dim_ok(d_v))
        return fail(KDA_ERR_UNSUPPORTED, "d_k and d_v must be 16, 32, 64 or 128 (got %d, %d)",
                    d_k, d_v);
    return KDA_OK;
}

struct Ptr {
    const void *p;
    const char *name;
    bool required;
    size_t align;     // bytes: the widest vector access the kernels make
};

kda_status check_ptrs(const Ptr *ps, int n)
{
    for (int i = 0; i < n; ++i) {
        if (!ps[i].p) {
            if (ps[i].required) return fail(KDA_ERR_INVALID_ARG, "%s is NULL", ps[i].name);
            continue;
        }
        if (!aligned(ps[i].p, ps[i].align))
            return fail(KDA_ERR_INVALID_ARG, "%s is not %zu-byte aligned", ps[i].name,
                        ps[i].align);
    }
    return KDA_OK;
}

bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
    return x < y + nb && y < x + na;
}

kda_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return ok();
    return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Size checks shared by kda_fwd_chunked and kda_fwd_workspace_bytes.
kda_status check_fwd_sizes(int32_t n_seqs, int64_t n_tokens, int32_t H, int32_t d_k,
                           int32_t d_v, bool packed)
{
    kda_status s;
    if ((s = check_dims(H, d_k, d_v)) != KDA_OK) return s;
    if (n_seqs < 0) return fail(KDA_ERR_INVALID_ARG, "n_seqs must be >= 0 (got %d)", n_seqs);
    if (n_tokens < 0) return fail(KDA_ERR_INVALID_ARG, "n_tokens must be >= 0");
    if (n_tokens > ((int64_t)1 << 31) - 64)
        return fail(KDA_ERR_INVALID_ARG,
                    "n_tokens must fit int32 with room for one chunk (cu_seqlens is int32)");
    if ((int64_t)H * (d_k > d_v ? d_k : d_v) >= ((int64_t)1 << 25))
        return fail(KDA_ERR_INVALID_ARG, "H * d must be below 2^25 (16 rows of a tensor "
                                         "must stay below 2^31 bytes)");
    if (n_seqs == 0 && n_tokens != 0)
        return fail(KDA_ERR_INVALID_ARG, "n_tokens > 0 with n_seqs == 0");
    if (n_seqs > 0 && !packed && n_tokens % n_seqs)
        return fail(KDA_ERR_INVALID_ARG,
                    "without cu_seqlens n_tokens (%lld) must be a multiple of n_seqs (%d)",
                    (long long)n_tokens, n_seqs);
    return KDA_OK;
}

kda::PrefillArgs size_args(int32_t n_seqs, int64_t n_tokens, int32_t H, int32_t d_k,
                           int32_t d_v, bool in_bf16, const int32_t *cu_seqlens)
{
    kda::PrefillArgs a{};
    a.cu_seqlens = cu_seqlens;
    a.n_seqs = n_seqs;
    a.n_tokens = n_tokens;
    a.seqlen = (!cu_seqlens && n_seqs > 0) ? (int32_t)(n_tokens / n_seqs) : 0;
    a.H = H; a.d_k = d_k; a.d_v = d_v;
    a.in_bf16 = in_bf16;
    return a;
}

constexpr size_t kWorkspaceAlign = 256;

}  // namespace

KDA_API size_t kda_fwd_workspace_bytes(int32_t n_seqs, int64_t n_tokens, int32_t H,
                                       int32_t d_k, int32_t d_v, kda_dtype in_dtype)
{
    if (in_dtype != KDA_F32 && in_dtype != KDA_BF16) return 0;
    if (check_fwd_sizes(n_seqs, n_tokens, H, d_k, d_v, false) != KDA_OK) return 0;
    if (n_seqs == 0 || n_tokens == 0) return 0;
    return kda::prefill_workspace_bytes(
        size_args(n_seqs, n_tokens, H, d_k, d_v, in_dtype == KDA_BF16, nullptr));
}

namespace {
// a non-null placeholder: only its being set matters to the size planner
const int32_t kPackedMarker = 0;
}  // namespace

namespace {

// Shared body of kda_fwd_chunked and kda_fwd_chunked_gated.  Gated: z and b
// (input type) and A_log replace g and beta, which are then unused.
kda_status fwd_impl(const char *fn, const void *q, const void *k, const void *v,
                    const float *g, const float *beta, const void *z, const float *A_log,
                    const void *b, bool gated, const float *S0, const int32_t *cu_seqlens,
                    int32_t n_seqs, int64_t n_tokens, int32_t H, int32_t d_k, int32_t d_v,
                    kda_dtype in_dtype, kda_dtype out_dtype, void *o, float *S_T,
                    void *workspace, size_t workspace_bytes, kda_stream_t stream)
{
    kda_status s;
    if ((s = check_dtypes(in_dtype, out_dtype)) != KDA_OK) return s;
    if ((s = check_fwd_sizes(n_seqs, n_tokens, H, d_k, d_v, cu_seqlens != nullptr)) != KDA_OK)
        return s;
    if (cu_seqlens && !aligned(cu_seqlens, 4))
        return fail(KDA_ERR_INVALID_ARG, "cu_seqlens is not 4-byte aligned");
    if (!workspace && workspace_bytes != 0)
        return fail(KDA_ERR_INVALID_ARG, "workspace is NULL but workspace_bytes is %zu",
                    workspace_bytes);
    if (workspace && !aligned(workspace, kWorkspaceAlign))
        return fail(KDA_ERR_INVALID_ARG, "workspace is not %zu-byte aligned", kWorkspaceAlign);
    if (gated && !A_log) return fail(KDA_ERR_INVALID_ARG, "A_log is NULL");
    if (n_seqs == 0) return ok();
    const int32_t seqlen = cu_seqlens ? 0 : (int32_t)(n_tokens / n_seqs);
    size_t need = 0;
    if (workspace) {
        need = kda::prefill_workspace_bytes(
            size_args(n_seqs, n_tokens, H, d_k, d_v, in_dtype == KDA_BF16,
                      cu_seqlens ? &kPackedMarker : nullptr));
        if (workspace_bytes < need)
            return fail(KDA_ERR_INVALID_ARG,
                        "workspace_bytes %zu is below the %zu bytes kda_fwd_workspace_bytes "
                        "gives for these sizes", workspace_bytes, need);
    }
    const bool have_tokens = n_tokens > 0;
    const size_t in_b = in_dtype == KDA_BF16 ? 2 : 4, out_b = out_dtype == KDA_BF16 ? 2 : 4;
    const Ptr ps[] = {{q, "q", have_tokens, 2 * in_b}, {k, "k", have_tokens, 2 * in_b},
                      {v, "v", have_tokens, 4 * in_b}, {o, "o", have_tokens, 4 * out_b},
                      {S0, "S0", false, 4}, {S_T, "S_T", false, 4},
                      {gated ? z : g, gated ? "z" : "g", have_tokens, gated ? 2 * in_b : 8},
                      {gated ? b : beta, gated ? "b" : "beta", have_tokens,
                       gated ? in_b : 4}, {A_log, "A_log", gated, 4}};
    if ((s = check_ptrs(ps, 9)) != KDA_OK) return s;
    const size_t o_bytes = (size_t)n_tokens * H * d_v * out_b;
    const size_t st_bytes = (size_t)n_seqs * H * d_k * d_v * 4;
    const size_t gb = gated ? in_b : 4;
    const void *ins[] = {q, k, v, gated ? z : g, gated ? b : beta, S0, gated ? A_log : nullptr};
    const size_t in_sz[] = {(size_t)n_tokens * H * d_k * in_b, (size_t)n_tokens * H * d_k * in_b,
                            (size_t)n_tokens * H * d_v * in_b, (size_t)n_tokens * H * d_k * gb,
                            (size_t)n_tokens * H * gb, st_bytes, (size_t)H * 4};
    for (int i = 0; i < 7; ++i) {
        if (overlap(o, o_bytes, ins[i], in_sz[i]) || overlap(S_T, st_bytes, ins[i], in_sz[i]))
            return fail(KDA_ERR_INVALID_ARG, "an output buffer overlaps an input buffer");
        if (overlap(workspace, need, ins[i], in_sz[i]))
            return fail(KDA_ERR_INVALID_ARG, "the workspace overlaps an input buffer");
    }
    if (overlap(o, o_bytes, S_T, st_bytes))
        return fail(KDA_ERR_INVALID_ARG, "o overlaps S_T");
    if (overlap(workspace, need, o, o_bytes) || overlap(workspace, need, S_T, st_bytes))
        return fail(KDA_ERR_INVALID_ARG, "the workspace overlaps an output buffer");

    kda::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S0 = S0;
    a.cu_seqlens = cu_seqlens; a.n_seqs = n_seqs; a.n_tokens = n_tokens; a.seqlen = seqlen;
    a.H = H; a.d_k = d_k; a.d_v = d_v;
    a.in_bf16 = in_dtype == KDA_BF16; a.out_bf16 = out_dtype == KDA_BF16;
    a.o = o; a.S_T = S_T; a.stream = stream;
    a.workspace = need ? workspace : nullptr;
    a.workspace_bytes = need;
    a.gated = gated; a.z = z; a.b = b; a.A_log = A_log;
    return hip_status(kda::launch_prefill(a), fn);
}

}  // namespace

KDA_API kda_status kda_fwd_chunked(const void *q, const void *k, const void *v,
                                   const float *g, const float *beta, const float *S0,
                                   const int32_t *cu_seqlens, int32_t n_seqs,
                                   int64_t n_tokens, int32_t H, int32_t d_k, int32_t d_v,
                                   kda_dtype in_dtype, kda_dtype out_dtype, void *o,
                                   float *S_T, void *workspace, size_t workspace_bytes,
                                   kda_stream_t stream)
{
    return fwd_impl("kda_fwd_chunked launch", q, k, v, g, beta, nullptr, nullptr, nullptr,
                    false, S0, cu_seqlens, n_seqs, n_tokens, H, d_k, d_v, in_dtype, out_dtype,
                    o, S_T, workspace, workspace_bytes, stream);
}

KDA_API kda_status kda_fwd_chunked_gated(const void *q, const void *k, const void *v,
                                         const void *z, const float *A_log, const void *b,
                                         const float *S0, const int32_t *cu_seqlens,
                                         int32_t n_seqs, int64_t n_tokens, int32_t H,
                                         int32_t d_k, int32_t d_v, kda_dtype in_dtype,
                                         kda_dtype out_dtype, void *o, float *S_T,
                                         void *workspace, size_t workspace_bytes,
                                         kda_stream_t stream)
{
    return fwd_impl("kda_fwd_chunked_gated launch", q, k, v, nullptr, nullptr, z, A_log, b,
                    true, S0, cu_seqlens, n_seqs, n_tokens, H, d_k, d_v, in_dtype, out_dtype,
                    o, S_T, workspace, workspace_bytes, stream);
}

KDA_API kda_status kda_decode_step(const void *q, const void *k, const void *v,
                                   const float *g, const float *beta, float *S,
                                   int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                                   kda_dtype in_dtype, kda_dtype out_dtype, void *o,
                                   kda_stream_t stream)
{
    kda_status s;
    if ((s = check_dtypes(in_dtype, out_dtype)) != KDA_OK) return s;
    if ((s = check_dims(H, d_k, d_v)) != KDA_OK) return s;
    if (N < 0) return fail(KDA_ERR_INVALID_ARG, "N must be >= 0 (got %d)", N);
    if (N == 0) return ok();
    const size_t in_b = in_dtype == KDA_BF16 ? 2 : 4, out_b = out_dtype == KDA_BF16 ? 2 : 4;
    const Ptr ps[] = {{q, "q", true, in_b}, {k, "k", true, in_b}, {v, "v", true, 4 * in_b},
                      {g, "g", true, 4}, {beta, "beta", true, 4}, {S, "S", true, 16},
                      {o, "o", true, 4 * out_b}};
    if ((s = check_ptrs(ps, 7)) != KDA_OK) return s;
    const size_t nh = (size_t)N * H;
    const size_t s_bytes = nh * d_k * d_v * 4;
    const void *others[] = {q, k, v, g, beta, o};
    const size_t sz[] = {nh * d_k * in_b, nh * d_k * in_b, nh * d_v * in_b, nh * d_k * 4,
                         nh * 4, nh * d_v * out_b};
    for (int i = 0; i < 6; ++i)
        if (overlap(S, s_bytes, others[i], sz[i]))
            return fail(KDA_ERR_INVALID_ARG, "S overlaps another argument");
    for (int i = 0; i < 5; ++i)
        if (overlap(o, sz[5], others[i], sz[i]))
            return fail(KDA_ERR_INVALID_ARG, "o overlaps an input");

    kda::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S = S; a.o = o;
    a.N = N; a.H = H; a.d_k = d_k; a.d_v = d_v;
    a.in_bf16 = in_dtype == KDA_BF16; a.out_bf16 = out_dtype == KDA_BF16;
    a.stream = stream;
    return hip_status(kda::launch_decode(a), "kda_decode_step launch");
}

namespace {

// Shared validation of the speculative-decoding calls.  Token tensors are
// [N, K, H, d] (one row of K tokens per sequence), the state [N, H, d_k, d_v].
kda_status check_spec(const char *fn, int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                      int32_t K, int32_t K_min, const char *kname)
{
    kda_status s;
    if ((s = check_dims(H, d_k, d_v)) != KDA_OK) return s;
    if (N < 0) return fail(KDA_ERR_INVALID_ARG, "%s: N must be >= 0 (got %d)", fn, N);
    if (K < K_min || K > kda::kSpecMaxTokens)
        return fail(KDA_ERR_INVALID_ARG, "%s: %s must be in [%d, %d] (got %d)", fn, kname, K_min,
                    kda::kSpecMaxTokens, K);
    return KDA_OK;
}

struct Span {
    const void *p;
    size_t bytes;
};

// true if one of the first nw spans (the written ones) overlaps any other
// span of the na
bool spans_overlap(const Span *all, int nw, int na)
{
    for (int i = 0; i < nw; ++i)
        for (int j = 0; j < na; ++j)
            if (j != i && overlap(all[i].p, all[i].bytes, all[j].p, all[j].bytes))
                return true;
    return false;
}

kda_status run_spec(kda::SpecArgs &a, const char *fn)
{
    return hip_status(kda::launch_spec(a), fn);
}

}  // namespace

KDA_API kda_status kda_decode_verify(const void *q, const void *k, const void *v,
                                     const float *g, const float *beta, const float *S,
                                     int32_t N, int32_t K, int32_t H, int32_t d_k, int32_t d_v,
                                     kda_dtype in_dtype, kda_dtype out_dtype, void *o,
                                     kda_stream_t stream)
{
    kda_status s;
    if ((s = check_dtypes(in_dtype, out_dtype)) != KDA_OK) return s;
    if ((s = check_spec("kda_decode_verify", N, H, d_k, d_v, K, 1, "K")) != KDA_OK) return s;
    if (N == 0) return ok();
    const size_t in_b = in_dtype == KDA_BF16 ? 2 : 4, out_b = out_dtype == KDA_BF16 ? 2 : 4;
    const Ptr ps[] = {{q, "q", true, in_b}, {k, "k", true, in_b}, {v, "v", true, 4 * in_b},
                      {g, "g", true, 4}, {beta, "beta", true, 4}, {S, "S", true, 16},
                      {o, "o", true, 4 * out_b}};
    if ((s = check_ptrs(ps, 7)) != KDA_OK) return s;
    const size_t nt = (size_t)N * K * H;
    const Span all[] = {{o, nt * d_v * out_b}, {q, nt * d_k * in_b}, {k, nt * d_k * in_b},
                        {v, nt * d_v * in_b}, {g, nt * d_k * 4}, {beta, nt * 4},
                        {S, (size_t)N * H * d_k * d_v * 4}};
    if (spans_overlap(all, 1, 7))
        return fail(KDA_ERR_INVALID_ARG, "kda_decode_verify: o overlaps an input");
    kda::SpecArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o; a.K = K;
    a.S = const_cast<float *>(S);         // read only: write_state is false
    a.N = N; a.H = H; a.d_k = d_k; a.d_v = d_v;
    a.in_bf16 = in_dtype == KDA_BF16; a.out_bf16 = out_dtype == KDA_BF16;
    a.write_state = false; a.stream = stream;
    return run_spec(a, "kda_decode_verify launch");
}

KDA_API kda_status kda_decode_commit(const void *k, const void *v, const float *g,
                                     const float *beta, const int32_t *n_accept, float *S,
                                     int32_t N, int32_t K, int32_t H, int32_t d_k, int32_t d_v,
                                     kda_dtype in_dtype, kda_stream_t stream)
{
    kda_status s;
    if ((s = check_dtypes(in_dtype, in_dtype)) != KDA_OK) return s;
    if ((s = check_spec("kda_decode_commit", N, H, d_k, d_v, K, 0, "K")) != KDA_OK) return s;
    if (N == 0 || K == 0) return ok();
    const size_t in_b = in_dtype == KDA_BF16 ? 2 : 4;
    const Ptr ps[] = {{k, "k", true, in_b}, {v, "v", true, 4 * in_b}, {g, "g", true, 4},
                      {beta, "beta", true, 4}, {n_accept, "n_accept", true, 4},
                      {S, "S", true, 16}};
    if ((s = check_ptrs(ps, 6)) != KDA_OK) return s;
    const size_t nt = (size_t)N * K * H;
    const Span all[] = {{S, (size_t)N * H * d_k * d_v * 4}, {k, nt * d_k * in_b},
                        {v, nt * d_v * in_b}, {g, nt * d_k * 4}, {beta, nt * 4},
                        {n_accept, (size_t)N * 4}};
    if (spans_overlap(all, 1, 6))
        return fail(KDA_ERR_INVALID_ARG, "kda_decode_commit: S overlaps another argument");
    kda::SpecArgs a{};
    a.rk = k; a.rv = v; a.rg = g; a.rbeta = beta; a.n_accept = n_accept; a.Kr = K;
    a.K = 0; a.S = S; a.N = N; a.H = H; a.d_k = d_k; a.d_v = d_v;
    a.in_bf16 = in_dtype == KDA_BF16; a.out_bf16 = a.in_bf16;
    a.write_state = true; a.stream = stream;
    return run_spec(a, "kda_decode_commit launch");
}

KDA_API kda_status kda_decode_spec(const void *k_prev, const void *v_prev, const float *g_prev,
                                   const float *beta_prev, const int32_t *n_accept,
                                   int32_t K_prev, const void *q, const void *k, const void *v,
                                   const float *g, const float *beta, int32_t K, float *S,
                                   int32_t N, int32_t H, int32_t d_k, int32_t d_v,
                                   kda_dtype in_dtype, kda_dtype out_dtype, void *o,
                                   kda_stream_t stream)
{
    kda_status s;
    if ((s = check_dtypes(in_dtype, out_dtype)) != KDA_OK) return s;
    if ((s = check_spec("kda_decode_spec", N, H, d_k, d_v, K, 1, "K")) != KDA_OK) return s;
    if (K_prev < 0 || K_prev > kda::kSpecMaxTokens)
        return fail(KDA_ERR_INVALID_ARG, "kda_decode_spec: K_prev must be in [0, %d] (got %d)",
                    kda::kSpecMaxTokens, K_prev);
    if (N == 0) return ok();
    const size_t in_b = in_dtype == KDA_BF16 ? 2 : 4, out_b = out_dtype == KDA_BF16 ? 2 : 4;
    const bool prev = K_prev > 0;
    const Ptr ps[] = {{q, "q", true, in_b}, {k, "k", true, in_b}, {v, "v", true, 4 * in_b},
                      {g, "g", true, 4}, {beta, "beta", true, 4}, {S, "S", true, 16},
                      {o, "o", true, 4 * out_b}, {k_prev, "k_prev", prev, in_b},
                      {v_prev, "v_prev", prev, 4 * in_b}, {g_prev, "g_prev", prev, 4},
                      {beta_prev, "beta_prev", prev, 4}, {n_accept, "n_accept", prev, 4}};
    if ((s = check_ptrs(ps, 12)) != KDA_OK) return s;
    const size_t nt = (size_t)N * K * H, np = (size_t)N * K_prev * H;
    const Span all[] = {{S, (size_t)N * H * d_k * d_v * 4}, {o, nt * d_v * out_b},
                        {q, nt * d_k * in_b}, {k, nt * d_k * in_b}, {v, nt * d_v * in_b},
                        {g, nt * d_k * 4}, {beta, nt * 4}, {k_prev, np * d_k * in_b},
                        {v_prev, np * d_v * in_b}, {g_prev, np * d_k * 4}, {beta_prev, np * 4},
                        {n_accept, prev ? (size_t)N * 4 : 0}};
    if (spans_overlap(all, 2, 12))
        return fail(KDA_ERR_INVALID_ARG, "kda_decode_spec: S or o overlaps another argument");
    kda::SpecArgs a{};
    if (prev) {
        a.rk = k_prev; a.rv = v_prev; a.rg = g_prev; a.rbeta = beta_prev;
        a.n_accept = n_accept; a.Kr = K_prev;
    }
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o; a.K = K;
    a.S = S; a.N = N; a.H = H; a.d_k = d_k; a.d_v = d_v;
    a.in_bf16 = in_dtype == KDA_BF16; a.out_bf16 = out_dtype == KDA_BF16;
    a.write_state = true; a.stream = stream;
    return run_spec(a, "kda_decode_spec launch");
}

namespace {

// chunk slots (bos / 16 + n + c) of a batch: an upper bound on every slot + 1
int64_t bwd_slots(int32_t n_seqs, int64_t n_tokens) { return n_tokens / 16 + n_seqs + 1; }

}  // namespace

KDA_API size_t kda_bwd_workspace_bytes(int32_t n_seqs, int64_t n_tokens, int32_t H, int32_t d_k,
                                       int32_t d_v)
{
    if (check_fwd_sizes(n_seqs, n_tokens, H, d_k, d_v, true) != KDA_OK) return 0;
    if (n_seqs == 0) return 0;
    const size_t slots = (size_t)bwd_slots(n_seqs, n_tokens);
    const size_t ck = slots * H * d_k * d_v * 4;
    const size_t part = slots * H * kda::bwd_part_floats(d_k, d_v) * 4;
    return ((ck + 255) & ~(size_t)255) + ((part + 255) & ~(size_t)255);
}

KDA_API kda_status kda_bwd_chunked(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *S0,
                                   const int32_t *cu_seqlens, int32_t n_seqs, int64_t n_tokens,
                                   int32_t H, int32_t d_k, int32_t d_v, kda_dtype in_dtype,
                                   const void *dO, const float *dS_T, float *dq, float *dk,
                                   float *dv, float *dg, float *dbeta, float *dS0,
                                   void *workspace, size_t workspace_bytes, kda_stream_t stream)
{
    kda_status s;
    if ((s = check_dtypes(in_dtype, in_dtype)) != KDA_OK) return s;
    if ((s = check_fwd_sizes(n_seqs, n_tokens, H, d_k, d_v, cu_seqlens != nullptr)) != KDA_OK)
        return s;
    if (cu_seqlens && !aligned(cu_seqlens, 4))
        return fail(KDA_ERR_INVALID_ARG, "cu_seqlens is not 4-byte aligned");
    if (n_seqs == 0) return ok();
    const size_t need = kda_bwd_workspace_bytes(n_seqs, n_tokens, H, d_k, d_v);
    if (!workspace) return fail(KDA_ERR_INVALID_ARG, "workspace is NULL");
    if (!aligned(workspace, kWorkspaceAlign))
        return fail(KDA_ERR_INVALID_ARG, "workspace is not %zu-byte aligned", kWorkspaceAlign);
    if (workspace_bytes < need)
        return fail(KDA_ERR_INVALID_ARG,
                    "workspace_bytes %zu is below the %zu bytes kda_bwd_workspace_bytes gives",
                    workspace_bytes, need);
    const bool tok = n_tokens > 0;
    const size_t in_b = in_dtype == KDA_BF16 ? 2 : 4;
    // alignment: the widest vector access the kernels make
    const Ptr ps[] = {{q, "q", tok, 2 * in_b}, {k, "k", tok, 2 * in_b},
                      {v, "v", tok, 4 * in_b}, {g, "g", tok, 8}, {beta, "beta", tok, 4},
                      {dO, "dO", tok, 4 * in_b}, {S0, "S0", false, 4},
                      {dS_T, "dS_T", false, 4}, {dq, "dq", tok, 16}, {dk, "dk", tok, 16},
                      {dv, "dv", tok, 4}, {dg, "dg", tok, 4}, {dbeta, "dbeta", tok, 4},
                      {dS0, "dS0", false, 4}};
    if ((s = check_ptrs(ps, 14)) != KDA_OK) return s;
    const size_t nk = (size_t)n_tokens * H * d_k, nv = (size_t)n_tokens * H * d_v;
    const size_t st = (size_t)n_seqs * H * d_k * d_v * 4;
    // written spans first: the gradients and the workspace
    const Span all[] = {{dq, nk * 4}, {dk, nk * 4}, {dv, nv * 4}, {dg, nk * 4},
                        {dbeta, (size_t)n_tokens * H * 4}, {dS0, st}, {workspace, need},
                        {q, nk * in_b}, {k, nk * in_b}, {v, nv * in_b}, {g, nk * 4},
                        {beta, (size_t)n_tokens * H * 4}, {dO, nv * in_b}, {S0, st},
                        {dS_T, st}};
    if (spans_overlap(all, 7, 15))
        return fail(KDA_ERR_INVALID_ARG, "kda_bwd_chunked: an output or the workspace overlaps "
                                         "another argument");
    char *ws = static_cast<char *>(workspace);
    const size_t slots = (size_t)bwd_slots(n_seqs, n_tokens);
    float *ckpt = reinterpret_cast<float *>(ws);
    float *part = reinterpret_cast<float *>(
        ws + ((slots * H * d_k * d_v * 4 + 255) & ~(size_t)255));
    const int32_t seqlen = cu_seqlens ? 0 : (int32_t)(n_tokens / n_seqs);
    // 1. the forward, keeping the state at every chunk start
    kda::PrefillArgs f{};
    f.q = q; f.k = k; f.v = v; f.g = g; f.beta = beta; f.S0 = S0;
    f.cu_seqlens = cu_seqlens; f.n_seqs = n_seqs; f.n_tokens = n_tokens; f.seqlen = seqlen;
    f.H = H; f.d_k = d_k; f.d_v = d_v;
    f.in_bf16 = in_dtype == KDA_BF16; f.out_bf16 = f.in_bf16;
    f.o = nullptr; f.S_T = nullptr; f.ckpt = ckpt; f.stream = stream;
    if ((s = hip_status(kda::launch_prefill(f), "kda_bwd_chunked forward launch")) != KDA_OK)
        return s;
    // 2. the reverse sweep and the per-chunk finish
    kda::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.dO = dO; a.g = g; a.beta = beta; a.dST = dS_T;
    a.cu_seqlens = cu_seqlens; a.n_seqs = n_seqs; a.n_tokens = n_tokens; a.seqlen = seqlen;
    a.H = H; a.d_k = d_k; a.d_v = d_v; a.in_bf16 = in_dtype == KDA_BF16;
    a.ckpt = ckpt; a.part = part; a.n_slots = (int64_t)slots;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dS0 = dS0;
    a.stream = stream;
    return hip_status(kda::launch_bwd(a), "kda_bwd_chunked launch");
}

KDA_API const char *kda_status_string(kda_status s)
{
    switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "KDA_ERR_UNKNOWN";
}

KDA_API const char *kda_last_error(void) { return g_err; }

kda_status kda::set_error(kda_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

KDA_API const char *kda_version(void) { return "0.1 gfx950"; }
