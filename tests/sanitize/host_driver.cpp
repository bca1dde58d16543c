// Host-only sanitizer driver (AddressSanitizer + UndefinedBehaviorSanitizer).
//
// Links the C-ABI layer (kda_api.cpp, compiled as plain host C++) against
// stub kernel launchers that record their arguments instead of touching a
// GPU, plus the fp64 C oracle, and walks every validation path of both entry
// points and the oracle's packed and single-chain calls.  Any out-of-bounds
// access, leak or undefined operation aborts the run with a sanitizer
// report; the pytest wrapper checks for a clean exit.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kda.h"
#include "kda_launch.h"

extern "C" {
int kda_oracle_fwd(const float *q, const float *k, const float *v, const float *g,
                   const float *beta, const float *S0, const int32_t *cu, int n_seqs, int H,
                   int dk, int dv, double *o, double *S_T, int n_threads);
void kda_oracle_head(int64_t T, int dk, int dv, const float *q, const float *k,
                     const float *v, const float *g, const float *beta, double *S, double *o);
}

namespace kda {
static int g_prefill_calls = 0, g_decode_calls = 0, g_spec_calls = 0, g_bwd_calls = 0;
static SpecArgs g_last_spec;
static PrefillArgs g_last_prefill;
size_t prefill_workspace_bytes(const PrefillArgs &a)
{
    // stand-in planner: scratch for one long sequence with few heads
    return (a.cu_seqlens == nullptr && a.seqlen >= 4096 && a.n_seqs * a.H <= 8) ? 1 << 20 : 0;
}
hipError_t launch_prefill(const PrefillArgs &a)
{
    ++g_prefill_calls;
    g_last_prefill = a;
    return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs &)
{
    ++g_decode_calls;
    return hipSuccess;
}
size_t bwd_part_floats(int32_t d_k, int32_t d_v) { return (size_t)d_k * d_v; }
hipError_t launch_bwd(const BwdArgs &)
{
    ++g_bwd_calls;
    return hipSuccess;
}
hipError_t launch_spec(const SpecArgs &a)
{
    ++g_spec_calls;
    g_last_spec = a;
    return hipSuccess;
}
}  // namespace kda

static int failures = 0;
#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            std::fprintf(stderr, "%s:%d: expectation failed: %s (last error: %s)\n", \
                         __FILE__, __LINE__, #cond, kda_last_error());            \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

int main()
{
    // device pointers are never dereferenced by the host layer: use
    // distinct, aligned host buffers so the overlap checks see real ranges
    const int64_t N = 4096;
    const int H = 2, D = 128;
    std::vector<uint16_t> q(N * H * D), k(N * H * D), v(N * H * D), o(N * H * D);
    std::vector<float> g(N * H * D), beta(N * H), S(2 * H * D * D), S0(2 * H * D * D);
    alignas(256) static unsigned char ws[(1 << 20) + 512];

    // valid calls reach the launcher
    EXPECT(kda_fwd_chunked(q.data(), k.data(), v.data(), g.data(), beta.data(), nullptr,
                           nullptr, 1, N, H, D, D, KDA_BF16, KDA_BF16, o.data(), S.data(),
                           nullptr, 0, nullptr) == KDA_OK);
    EXPECT(kda::g_prefill_calls == 1 && kda::g_last_prefill.workspace == nullptr);
    EXPECT(kda_fwd_chunked(q.data(), k.data(), v.data(), g.data(), beta.data(), S0.data(),
                           nullptr, 1, N, H, D, D, KDA_BF16, KDA_BF16, o.data(), S.data(), ws,
                           1 << 20, nullptr) == KDA_OK);
    EXPECT(kda::g_last_prefill.workspace == ws && kda::g_last_prefill.seqlen == N);
    // invalid calls are rejected before any launch
    const int before = kda::g_prefill_calls;
    EXPECT(kda_fwd_chunked(nullptr, k.data(), v.data(), g.data(), beta.data(), nullptr,
                           nullptr, 1, N, H, D, D, KDA_BF16, KDA_BF16, o.data(), S.data(),
                           nullptr, 0, nullptr) == KDA_ERR_INVALID_ARG);
    EXPECT(kda_fwd_chunked(q.data(), k.data(), v.data(), g.data(), beta.data(), nullptr,
                           nullptr, 1, N, H, 48, D, KDA_BF16, KDA_BF16, o.data(), S.data(),
                           nullptr, 0, nullptr) == KDA_ERR_UNSUPPORTED);
    EXPECT(kda_fwd_chunked(q.data(), k.data(), v.data(), g.data(), beta.data(), nullptr,
                           nullptr, 3, N, H, D, D, KDA_BF16, KDA_BF16, o.data(), S.data(),
                           nullptr, 0, nullptr) == KDA_ERR_INVALID_ARG);
    EXPECT(kda_fwd_chunked(q.data(), k.data(), v.data(), g.data(), beta.data(), nullptr,
                           nullptr, 1, N, H, D, D, KDA_BF16, KDA_BF16, q.data(), S.data(),
                           nullptr, 0, nullptr) == KDA_ERR_INVALID_ARG);   // o overlaps q
    EXPECT(kda_fwd_chunked(q.data(), k.data(), v.data(), g.data(), beta.data(), nullptr,
                           nullptr, 1, N, H, D, D, KDA_BF16, KDA_BF16, o.data(), S.data(), ws,
                           1 << 10, nullptr) == KDA_ERR_INVALID_ARG);      // too small
    EXPECT(kda_fwd_chunked(q.data(), k.data(), v.data(), g.data(), beta.data(), nullptr,
                           nullptr, 1, N, H, D, D, KDA_BF16, KDA_BF16, o.data(), S.data(),
                           ws + 64, 1 << 20, nullptr) == KDA_ERR_INVALID_ARG);  // misaligned
    EXPECT(kda_fwd_chunked(q.data(), k.data(), v.data(), g.data(), beta.data(), nullptr,
                           nullptr, 1, N, H, D, D, KDA_BF16, KDA_BF16, o.data(), S.data(),
                           nullptr, 4096, nullptr) == KDA_ERR_INVALID_ARG);   // NULL, bytes
    EXPECT(kda_fwd_chunked(q.data(), k.data(), v.data(), g.data(), beta.data(), nullptr,
                           nullptr, 1, (int64_t)1 << 31, H, D, D, KDA_BF16, KDA_BF16, o.data(),
                           S.data(), nullptr, 0, nullptr) == KDA_ERR_INVALID_ARG);
    EXPECT(kda_fwd_chunked(q.data(), k.data(), v.data(), g.data(), beta.data(), nullptr,
                           nullptr, 1, N, H, D, D, (kda_dtype)9, KDA_BF16, o.data(), S.data(),
                           nullptr, 0, nullptr) == KDA_ERR_INVALID_ARG);
    // the gated prologue variant: z as q, b one element per (token, head)
    std::vector<uint16_t> z(N * H * D), bb(N * H);
    std::vector<float> A_log(H);
    EXPECT(kda_fwd_chunked_gated(q.data(), k.data(), v.data(), z.data(), A_log.data(),
                                 bb.data(), nullptr, nullptr, 1, N, H, D, D, KDA_BF16, KDA_BF16,
                                 o.data(), S.data(), nullptr, 0, nullptr) == KDA_OK);
    EXPECT(kda::g_last_prefill.gated && kda::g_last_prefill.z == z.data());
    EXPECT(kda_fwd_chunked_gated(q.data(), k.data(), v.data(), z.data(), nullptr, bb.data(),
                                 nullptr, nullptr, 1, N, H, D, D, KDA_BF16, KDA_BF16, o.data(),
                                 S.data(), nullptr, 0, nullptr) == KDA_ERR_INVALID_ARG);
    EXPECT(kda_fwd_chunked_gated(q.data(), k.data(), v.data(), z.data(), A_log.data(),
                                 bb.data(), nullptr, nullptr, 1, N, H, D, D, KDA_BF16, KDA_BF16,
                                 z.data(), S.data(), nullptr, 0, nullptr) == KDA_ERR_INVALID_ARG);
    EXPECT(kda::g_prefill_calls == before + 1);
    EXPECT(std::strlen(kda_last_error()) > 0);
    EXPECT(kda_fwd_workspace_bytes(1, N, H, D, D, KDA_BF16) == (size_t)1 << 20);
    EXPECT(kda_fwd_workspace_bytes(-1, N, H, D, D, KDA_BF16) == 0);

    // decode
    EXPECT(kda_decode_step(q.data(), k.data(), v.data(), g.data(), beta.data(), S.data(), 2, H,
                           D, D, KDA_BF16, KDA_BF16, o.data(), nullptr) == KDA_OK);
    EXPECT(kda::g_decode_calls == 1);
    EXPECT(kda_decode_step(q.data(), k.data(), v.data(), g.data(), beta.data(), S.data(), -1,
                           H, D, D, KDA_BF16, KDA_BF16, o.data(), nullptr) == KDA_ERR_INVALID_ARG);
    EXPECT(kda_decode_step(q.data(), k.data(), v.data(), g.data(), beta.data(),
                           reinterpret_cast<float *>(q.data()), 1, 1, 16, 16, KDA_BF16, KDA_BF16,
                           o.data(), nullptr) == KDA_ERR_INVALID_ARG);      // S overlaps q
    // speculative decoding: [N = 2, K = 4, H, D] drafts fit in the token buffers
    std::vector<int32_t> acc(2, 3);
    EXPECT(kda_decode_verify(q.data(), k.data(), v.data(), g.data(), beta.data(), S.data(), 2, 4,
                             H, D, D, KDA_BF16, KDA_BF16, o.data(), nullptr) == KDA_OK);
    EXPECT(kda::g_last_spec.write_state == false && kda::g_last_spec.K == 4);
    EXPECT(kda_decode_commit(k.data(), v.data(), g.data(), beta.data(), acc.data(), S.data(), 2,
                             4, H, D, D, KDA_BF16, nullptr) == KDA_OK);
    EXPECT(kda::g_last_spec.write_state && kda::g_last_spec.K == 0 && kda::g_last_spec.Kr == 4);
    EXPECT(kda_decode_spec(k.data(), v.data(), g.data(), beta.data(), acc.data(), 4, q.data(),
                           k.data(), v.data(), g.data(), beta.data(), 4, S.data(), 2, H, D, D,
                           KDA_BF16, KDA_BF16, o.data(), nullptr) == KDA_OK);
    EXPECT(kda::g_spec_calls == 3);
    EXPECT(kda_decode_verify(q.data(), k.data(), v.data(), g.data(), beta.data(), S.data(), 2,
                             17, H, D, D, KDA_BF16, KDA_BF16, o.data(), nullptr) ==
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_decode_verify(q.data(), k.data(), v.data(), g.data(), beta.data(), S.data(), 2, 4,
                             H, D, D, KDA_BF16, KDA_BF16, q.data(), nullptr) ==
           KDA_ERR_INVALID_ARG);                                          // o overlaps q
    EXPECT(kda_decode_commit(k.data(), v.data(), g.data(), beta.data(), nullptr, S.data(), 2, 4,
                             H, D, D, KDA_BF16, nullptr) == KDA_ERR_INVALID_ARG);
    EXPECT(kda::g_spec_calls == 3);
    // backward: the forward with checkpoints, then the sweep and finish
    {
        std::vector<float> gq(N * H * D), gk(N * H * D), gv(N * H * D), gg(N * H * D),
            gb(N * H);
        const size_t need = kda_bwd_workspace_bytes(1, N, H, D, D);
        std::vector<unsigned char> wsb(need + 256);
        void *wsp = reinterpret_cast<void *>(
            (reinterpret_cast<uintptr_t>(wsb.data()) + 255) & ~(uintptr_t)255);
        const int pf = kda::g_prefill_calls;
        EXPECT(kda_bwd_chunked(q.data(), k.data(), v.data(), g.data(), beta.data(), nullptr,
                               nullptr, 1, N, H, D, D, KDA_BF16, o.data(), nullptr, gq.data(),
                               gk.data(), gv.data(), gg.data(), gb.data(), nullptr, wsp, need,
                               nullptr) == KDA_OK);
        EXPECT(kda::g_prefill_calls == pf + 1 && kda::g_last_prefill.ckpt != nullptr &&
               kda::g_last_prefill.o == nullptr && !kda::g_last_prefill.gated &&
               kda::g_bwd_calls == 1);
        EXPECT(kda_bwd_chunked(q.data(), k.data(), v.data(), g.data(), beta.data(), nullptr,
                               nullptr, 1, N, H, D, D, KDA_BF16, o.data(), nullptr, gq.data(),
                               gq.data(), gv.data(), gg.data(), gb.data(), nullptr, wsp, need,
                               nullptr) == KDA_ERR_INVALID_ARG);          // dk overlaps dq
        EXPECT(kda::g_bwd_calls == 1);
    }
    EXPECT(std::strcmp(kda_status_string(KDA_ERR_HIP), "KDA_ERR_HIP") == 0);
    EXPECT(std::strcmp(kda_status_string((kda_status)42), "KDA_ERR_UNKNOWN") == 0);
    EXPECT(std::strstr(kda_version(), "gfx950") != nullptr);

    // the oracle on a small packed batch, and one chain alone
    const int T0 = 37, T1 = 0, T2 = 21, Hn = 3, dk = 16, dv = 32, Nt = T0 + T1 + T2;
    std::vector<float> oq(Nt * Hn * dk), ok(Nt * Hn * dk), og(Nt * Hn * dk), ov(Nt * Hn * dv),
        ob(Nt * Hn), os0(3 * Hn * dk * dv);
    unsigned s = 12345;
    auto rnd = [&]() { s = s * 1103515245u + 12345u; return ((s >> 8) & 0xffff) / 65536.0f - 0.5f; };
    for (auto &x : oq) x = rnd();
    for (auto &x : ok) x = rnd();
    for (auto &x : ov) x = rnd();
    for (auto &x : og) x = -2.5f - 4.0f * rnd();
    for (auto &x : ob) x = 0.5f + rnd();
    for (auto &x : os0) x = rnd();
    const int32_t cu[4] = {0, T0, T0 + T1, Nt};
    std::vector<double> oo(Nt * Hn * dv), oS(3 * Hn * dk * dv);
    EXPECT(kda_oracle_fwd(oq.data(), ok.data(), ov.data(), og.data(), ob.data(), os0.data(), cu,
                          3, Hn, dk, dv, oo.data(), oS.data(), 2) >= 1);
    // sequence 2, head 1 alone must match the packed run
    std::vector<float> hq(T2 * dk), hk(T2 * dk), hg(T2 * dk), hv(T2 * dv), hb(T2);
    for (int t = 0; t < T2; ++t) {
        const int row = (T0 + T1 + t) * Hn + 1;
        std::memcpy(&hq[t * dk], &oq[row * dk], dk * 4);
        std::memcpy(&hk[t * dk], &ok[row * dk], dk * 4);
        std::memcpy(&hg[t * dk], &og[row * dk], dk * 4);
        std::memcpy(&hv[t * dv], &ov[row * dv], dv * 4);
        hb[t] = ob[row];
    }
    std::vector<double> hS(dk * dv), ho(T2 * dv);
    for (int e = 0; e < dk * dv; ++e) hS[e] = os0[(2 * Hn + 1) * dk * dv + e];
    kda_oracle_head(T2, dk, dv, hq.data(), hk.data(), hv.data(), hg.data(), hb.data(), hS.data(),
                    ho.data());
    double dmax = 0;
    for (int e = 0; e < dk * dv; ++e) {
        const double d = hS[e] - oS[(2 * Hn + 1) * dk * dv + e];
        dmax = d > dmax ? d : (-d > dmax ? -d : dmax);
    }
    EXPECT(dmax == 0.0);
    if (failures) return 1;
    std::printf("sanitized host checks passed\n");
    return 0;
}
