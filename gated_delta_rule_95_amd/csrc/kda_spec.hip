// KDA speculative decoding: verify K drafted tokens without advancing the
// state, and replay the accepted prefix into the state later.
//
// The KDA state is updated in place at decode, so when verification rejects
// some drafted tokens the state has already moved past the last accepted
// one; a snapshot per draft position would allow a rollback but multiplies
// the state traffic.  K3 instead keeps only each draft's inputs and replays
// the accepted ones on chip to rebuild the state (K3-on-TPU essay,
// blog.higcp.com, "KDA + Gated MLA", the costs section, item (1)).  Here:
//
//   verify  reads S (never writes it), runs the K drafts in registers and
//           writes o for every draft position;
//   commit  reads S, replays the first n_accept[n] cached tokens of each
//           sequence and writes S back;
//   spec    both in one pass: replay the previous step's accepted drafts,
//           write S, then run the new drafts and write their outputs.  The
//           state is read once and written once per step, the traffic of a
//           plain decode step, whatever K.
//
// Each token applies the KDA update of the Kimi K3 architecture walkthrough
// (mhpq.cn/news/56770, "KDA 到底在算什么"): S' = Diag(exp(g)) S,
// u = beta (v - S'^T k), S = S' + k u^T, o = S^T q = S'^T q + u (k . q).
// The thread tiling is the decode step's: one workgroup per (sequence,
// head), each thread four consecutive columns of R rows, the state in
// registers for all tokens.  Every token's per-channel vectors are staged in
// LDS before the first token, so the per-token work is the row pass, one
// column reduction and the rank-1 write.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <int DK, int DV>
struct SpecShape {
    static constexpr int NT = (DK * DV / 16) < 1024 ? (DK * DV / 16) : 1024;
    static constexpr int CB = DV / 4;           // 4-column blocks per row
    static constexpr int RP = NT / CB;          // rows covered per pass
    static constexpr int R = DK / RP;           // rows per thread
    static constexpr int NWV = NT / WAVE;
    static_assert(NT % CB == 0 && DK % RP == 0, "spec tiling");
};

template <typename TI, typename TO>
struct SpecParams {
    // replayed tokens [N, Kr, H, d] (k, v, g, beta), n_accept[N] of them
    const TI *rk, *rv;
    const float *rg, *rb;
    const int32_t *n_accept;
    int32_t Kr;
    // drafts [N, K, H, d] and their outputs
    const TI *q, *k, *v;
    const float *g, *b;
    TO *o;
    int32_t K;
    float *S;
    int32_t H;
    bool write_state;
};

template <int DK, int DV>
struct SpecSmem {
    float a[2][kSpecMaxTokens][DK];             // exp(g): replayed, drafts
    float k[2][kSpecMaxTokens][DK];
    float q[kSpecMaxTokens][DK];
    float v[2][kSpecMaxTokens][DV];
    float b[2][kSpecMaxTokens];
    // column reduction: per-wave partial sums (two-stage, d_v = 128) or per
    // row pass (other widths), and the broadcast delta u
    f32x4 wk[SpecShape<DK, DV>::NWV][32], wq[SpecShape<DK, DV>::NWV][32];
    float wkq[SpecShape<DK, DV>::NWV];
    static constexpr int RPX = SpecShape<DK, DV>::CB == 32 ? 1 : SpecShape<DK, DV>::RP;
    f32x4 pk[RPX][SpecShape<DK, DV>::CB];
    f32x4 pq[RPX][SpecShape<DK, DV>::CB];
    float kq[RPX];
    f32x4 u[DV / 4];
};

// One token on the register-held state: decay, the column sums S'^T k (and
// S'^T q, k . q when an output is wanted), u, the output, the rank-1 write.
template <bool WANT_O, typename TO, int DK, int DV>
__device__ __forceinline__ void spec_token(int tid, SpecSmem<DK, DV> &sm,
                                           f32x4 (&s)[SpecShape<DK, DV>::R], const float *a,
                                           const float *kv, const float *qv, const float *vv_,
                                           float b, TO *o)
{
    using Sh = SpecShape<DK, DV>;
    const int cb = tid % Sh::CB, r0 = tid / Sh::CB;
    f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f;
#pragma unroll
    for (int p = 0; p < Sh::R; ++p) {
        const int i = r0 + p * Sh::RP;
        const float ki = kv[i];
        s[p] *= a[i];
        pk += s[p] * ki;
        if constexpr (WANT_O) {
            const float qi = qv[i];
            pq += s[p] * qi;
            kq += ki * qi;
        }
    }
    const f32x4 vv = *reinterpret_cast<const f32x4 *>(vv_ + 4 * cb);
    if constexpr (Sh::CB == 32) {
        // the two 32-lane halves of a wave hold the same columns: one
        // register swap adds them; then two waves add the per-wave sums
        const int w = tid / WAVE, l = tid % WAVE;
        f32x4 wk, wq;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float lo, hi;
            half_pair(pk[e], lo, hi);
            wk[e] = lo + hi;
            if constexpr (WANT_O) {
                half_pair(pq[e], lo, hi);
                wq[e] = lo + hi;
            }
        }
        if (l < 32) {
            sm.wk[w][l] = wk;
            if constexpr (WANT_O) sm.wq[w][l] = wq;
        }
        if constexpr (WANT_O) {
            float klo, khi;
            half_pair(kq, klo, khi);
            if (l == 0) sm.wkq[w] = klo + khi;
        }
        __syncthreads();
        // u from the k sums on wave 0 (its two halves each add half of the
        // waves' partials, one register swap joins them); the output's sums
        // on wave 1, whose output waits for u after the next barrier
        constexpr int HW = Sh::NWV / 2;
        static_assert(Sh::NWV % 2 == 0 && Sh::NWV >= 2, "two halves of the per-wave sums");
        const int hh = l >> 5, c = l & 31;
        if (w == 0) {
            f32x4 ks = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < HW; ++r) ks += sm.wk[hh * HW + r][c];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float lo, hi;
                half_pair(ks[e], lo, hi);
                ks[e] = lo + hi;
            }
            if (hh == 0) sm.u[c] = b * (vv - ks);
        }
        f32x4 qs = {0.f, 0.f, 0.f, 0.f};
        float kqt = 0.f;
        if constexpr (WANT_O) {
            if (w == 1) {
#pragma unroll
                for (int r = 0; r < HW; ++r) {
                    qs += sm.wq[hh * HW + r][c];
                    kqt += sm.wkq[hh * HW + r];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float lo, hi;
                    half_pair(qs[e], lo, hi);
                    qs[e] = lo + hi;
                }
                float lo, hi;
                half_pair(kqt, lo, hi);
                kqt = lo + hi;
            }
        }
        __syncthreads();
        if constexpr (WANT_O) {
            if (w == 1 && hh == 0) Elem<TO>::st4(o + 4 * c, qs + sm.u[c] * kqt);
        }
        const f32x4 u = sm.u[cb];
#pragma unroll
        for (int p = 0; p < Sh::R; ++p) s[p] += kv[r0 + p * Sh::RP] * u;
        return;
    } else {
        sm.pk[r0][cb] = pk;
        if constexpr (WANT_O) {
            sm.pq[r0][cb] = pq;
            if (cb == 0) sm.kq[r0] = kq;
        }
        __syncthreads();
        if (r0 == 0) {
            f32x4 ks = {0.f, 0.f, 0.f, 0.f}, qs = {0.f, 0.f, 0.f, 0.f};
            float kqt = 0.f;
#pragma unroll
            for (int r = 0; r < Sh::RP; ++r) {
                ks += sm.pk[r][cb];
                if constexpr (WANT_O) {
                    qs += sm.pq[r][cb];
                    kqt += sm.kq[r];
                }
            }
            const f32x4 uu = b * (vv - ks);
            sm.u[cb] = uu;
            if constexpr (WANT_O) Elem<TO>::st4(o + 4 * cb, qs + uu * kqt);
        }
    }
    __syncthreads();
    const f32x4 u = sm.u[cb];
#pragma unroll
    for (int p = 0; p < Sh::R; ++p) s[p] += kv[r0 + p * Sh::RP] * u;
    // the next token's partial sums and u overwrite this token's only after
    // its own first barrier, which every thread reaches after reading u
}

// A workgroup's tokens are a chain of barriers and column reductions, so two
// workgroups per compute unit overlap each other's waits: at 1024 threads
// that needs 8 waves per SIMD, at most 64 VGPRs (the LDS holds two).
template <typename TI, typename TO, int DK, int DV>
__global__ __launch_bounds__((SpecShape<DK, DV>::NT), (SpecShape<DK, DV>::NT >= 1024 ? 8 : 1))
void kda_spec_kernel(const SpecParams<TI, TO> p)
{
    using Sh = SpecShape<DK, DV>;
    __shared__ SpecSmem<DK, DV> sm;
    const int tid = threadIdx.x;
    const int cb = tid % Sh::CB, r0 = tid / Sh::CB;
    const int64_t nh = blockIdx.x;               // n * H + h
    const int n = (int)(nh / p.H), h = (int)(nh % p.H);
    float *Sp = p.S + nh * (int64_t)(DK * DV);

    f32x4 s[Sh::R];
#pragma unroll
    for (int i = 0; i < Sh::R; ++i)
        s[i] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4 *>(Sp + (r0 + i * Sh::RP) * DV + 4 * cb));

    // accepted count, clamped into [0, Kr]: a value out of its contract
    // changes the result, never the addresses touched
    int nrep = 0;
    if (p.n_accept) {
        const int32_t na = p.n_accept[n];
        nrep = na < 0 ? 0 : (na > p.Kr ? p.Kr : na);
    }
    nrep = __builtin_amdgcn_readfirstlane(nrep);
    const int nd = p.K;

    // stage every token's vectors
    for (int e = tid; e < nrep * DK; e += Sh::NT) {
        const int t = e / DK, i = e % DK;
        const int64_t off = (((int64_t)n * p.Kr + t) * p.H + h) * DK + i;
        sm.a[0][t][i] = fast_exp2(p.rg[off] * LOG2E);
        sm.k[0][t][i] = Elem<TI>::ld(p.rk + off);
    }
    for (int e = tid; e < nrep * DV; e += Sh::NT) {
        const int t = e / DV, j = e % DV;
        sm.v[0][t][j] = Elem<TI>::ld(p.rv + (((int64_t)n * p.Kr + t) * p.H + h) * DV + j);
    }
    if (tid < nrep) sm.b[0][tid] = p.rb[((int64_t)n * p.Kr + tid) * p.H + h];
    for (int e = tid; e < nd * DK; e += Sh::NT) {
        const int t = e / DK, i = e % DK;
        const int64_t off = (((int64_t)n * nd + t) * p.H + h) * DK + i;
        sm.a[1][t][i] = fast_exp2(p.g[off] * LOG2E);
        sm.k[1][t][i] = Elem<TI>::ld(p.k + off);
        sm.q[t][i] = Elem<TI>::ld(p.q + off);
    }
    for (int e = tid; e < nd * DV; e += Sh::NT) {
        const int t = e / DV, j = e % DV;
        sm.v[1][t][j] = Elem<TI>::ld(p.v + (((int64_t)n * nd + t) * p.H + h) * DV + j);
    }
    if (tid < nd) sm.b[1][tid] = p.b[((int64_t)n * nd + tid) * p.H + h];
    __syncthreads();

    // replay the accepted tokens into the state
#pragma unroll 1
    for (int t = 0; t < nrep; ++t)
        spec_token<false, TO, DK, DV>(tid, sm, s, sm.a[0][t], sm.k[0][t], nullptr, sm.v[0][t],
                                      sm.b[0][t], nullptr);
    if (p.write_state) {
#pragma unroll
        for (int i = 0; i < Sh::R; ++i)
            __builtin_nontemporal_store(
                s[i], reinterpret_cast<f32x4 *>(Sp + (r0 + i * Sh::RP) * DV + 4 * cb));
    }
    // the drafts: outputs only, the state is not written
#pragma unroll 1
    for (int t = 0; t < nd; ++t)
        spec_token<true, TO, DK, DV>(tid, sm, s, sm.a[1][t], sm.k[1][t], sm.q[t], sm.v[1][t],
                                     sm.b[1][t], p.o + (((int64_t)n * nd + t) * p.H + h) * DV);
}

template <typename TI, typename TO, int DK, int DV>
static hipError_t launch_spec_t(const SpecArgs &a)
{
    using Sh = SpecShape<DK, DV>;
    const int64_t heads = (int64_t)a.N * a.H;
    if (heads == 0) return hipSuccess;
    if (heads * Sh::NT >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
    static_assert(sizeof(SpecSmem<DK, DV>) <= 160 * 1024, "LDS");
    SpecParams<TI, TO> p{};
    p.rk = (const TI *)a.rk; p.rv = (const TI *)a.rv; p.rg = a.rg; p.rb = a.rbeta;
    p.n_accept = a.n_accept; p.Kr = a.Kr;
    p.q = (const TI *)a.q; p.k = (const TI *)a.k; p.v = (const TI *)a.v;
    p.g = a.g; p.b = a.beta; p.o = (TO *)a.o; p.K = a.K;
    p.S = a.S; p.H = a.H; p.write_state = a.write_state;
    hipLaunchKernelGGL((kda_spec_kernel<TI, TO, DK, DV>), dim3((unsigned)heads), dim3(Sh::NT), 0,
                       (hipStream_t)a.stream, p);
    return hipGetLastError();
}

template <typename TI, typename TO>
static hipError_t dispatch_spec(const SpecArgs &a)
{
#define KDA_SPEC_CASE(DK_, DV_) \
    if (a.d_k == DK_ && a.d_v == DV_) return launch_spec_t<TI, TO, DK_, DV_>(a);
    KDA_SPEC_CASE(16, 16) KDA_SPEC_CASE(16, 32) KDA_SPEC_CASE(16, 64) KDA_SPEC_CASE(16, 128)
    KDA_SPEC_CASE(32, 16) KDA_SPEC_CASE(32, 32) KDA_SPEC_CASE(32, 64) KDA_SPEC_CASE(32, 128)
    KDA_SPEC_CASE(64, 16) KDA_SPEC_CASE(64, 32) KDA_SPEC_CASE(64, 64) KDA_SPEC_CASE(64, 128)
    KDA_SPEC_CASE(128, 16) KDA_SPEC_CASE(128, 32) KDA_SPEC_CASE(128, 64) KDA_SPEC_CASE(128, 128)
#undef KDA_SPEC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_spec(const SpecArgs &a)
{
    if (a.in_bf16) return a.out_bf16 ? dispatch_spec<bf16, bf16>(a) : dispatch_spec<bf16, float>(a);
    return dispatch_spec<float, float>(a);
}

}  // namespace kda
