// KDA decode step: one token per (sequence, head), state updated in place.
//
// Per (n, h), with S the d_k x d_v fp32 state (rows = key channels):
//     S' = Diag(exp(g)) S
//     u  = beta (v - S'^T k)
//     S  = S' + k u^T                  (written back in place)
//     o  = S^T q = S'^T q + u (k . q)
// which is the KDA update of the Kimi K3 architecture walkthrough
// (mhpq.cn/news/56770, "KDA 到底在算什么": state-update equation and the
// decay -> erase -> write order of its figure caption), applied once.
//
// The step is a pure stream over the state (64 KiB per head at d = 128,
// read once and written once), so it is built for HBM bandwidth: one
// workgroup per (n, h); each thread owns 4 consecutive columns of R = 4 rows
// and issues its four 16-byte state loads before doing anything else.
// State loads and stores are nontemporal: the state is touched once per
// step, so keeping it out of the caches leaves them to the small vectors.
// Both column reductions (S'^T k and S'^T q) share one pass over the rows
// and one LDS exchange; the o = S'^T q + u (k . q) identity removes the
// second pass the read would otherwise need.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <int DK, int DV>
struct DecodeShape {
    // threads: four 16-byte state loads each (R = 4 at every supported
    // shape; 1024 threads at d_k = d_v = 128).  On gfx950 this streamed the
    // state 6% faster than 256 threads with sixteen loads each.
    static constexpr int NT = (DK * DV / 16) < 1024 ? (DK * DV / 16) : 1024;
    static constexpr int CB = DV / 4;           // 4-column blocks per row
    static constexpr int RP = NT / CB;          // rows covered per pass
    static constexpr int R = DK / RP;           // rows per thread
    static_assert(NT % CB == 0 && DK % RP == 0, "decode tiling");
};

template <typename TI, typename TO, int DK, int DV>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT))
void kda_decode_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                       const TI *__restrict__ v, const float *__restrict__ g,
                       const float *__restrict__ beta, float *__restrict__ S,
                       TO *__restrict__ o)
{
    using Sh = DecodeShape<DK, DV>;
    const int tid = threadIdx.x;
    const int cb = tid % Sh::CB;
    const int r0 = tid / Sh::CB;
    const int64_t nh = blockIdx.x;           // (n * H + h): flat head index

    float *Sh_ = S + nh * (int64_t)(DK * DV);

    // 1. issue every state load first
    f32x4 s[Sh::R];
#pragma unroll
    for (int p = 0; p < Sh::R; ++p)
        s[p] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4 *>(Sh_ + (r0 + p * Sh::RP) * DV + 4 * cb));

    // 2. per-channel vectors into LDS
    __shared__ float s_a[DK], s_k[DK], s_q[DK];
    for (int i = tid; i < DK; i += Sh::NT) {
        s_a[i] = fast_exp2(g[nh * DK + i] * LOG2E);
        s_k[i] = Elem<TI>::ld(k + nh * DK + i);
        s_q[i] = Elem<TI>::ld(q + nh * DK + i);
    }
    const f32x4 vv = Elem<TI>::ld4(v + nh * DV + 4 * cb);
    const float b = beta[nh];
    __syncthreads();

    // 3. decay the rows, accumulate the two column partial sums
    f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f;
#pragma unroll
    for (int p = 0; p < Sh::R; ++p) {
        const int i = r0 + p * Sh::RP;
        const float a = s_a[i], ki = s_k[i], qi = s_q[i];
        s[p] *= a;
        pk += s[p] * ki;
        pq += s[p] * qi;
        kq += ki * qi;
    }
    // 4. column sums of the partials, delta u = beta (v - S'^T k), o
    f32x4 u;
    if constexpr (Sh::CB == 32) {
        // The two 32-lane halves of a wave hold the same columns (rows r0
        // and r0 + 1): one register swap adds them.  One half wave then adds
        // the per-wave sums, writes o and publishes u.  Compared with every
        // thread adding all RP row partials from LDS, this cuts the LDS
        // reads about twelvefold.
        constexpr int NWV = Sh::NT / WAVE;
        __shared__ f32x4 s_wk[NWV][32], s_wq[NWV][32], s_u[32];
        __shared__ float s_wkq[NWV];
        const int w = tid / WAVE, l = tid % WAVE;
        f32x4 wk, wq;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float lo, hi;
            half_pair(pk[e], lo, hi);
            wk[e] = lo + hi;
            half_pair(pq[e], lo, hi);
            wq[e] = lo + hi;
        }
        float klo, khi;
        half_pair(kq, klo, khi);
        if (l < 32) {
            s_wk[w][l] = wk;
            s_wq[w][l] = wq;
        }
        if (l == 0) s_wkq[w] = klo + khi;
        __syncthreads();
        if (tid < 32) {                  // cb == tid
            f32x4 ks = {0.f, 0.f, 0.f, 0.f}, qs = {0.f, 0.f, 0.f, 0.f};
            float kqt = 0.f;
#pragma unroll
            for (int r = 0; r < NWV; ++r) {
                ks += s_wk[r][tid];
                qs += s_wq[r][tid];
                kqt += s_wkq[r];
            }
            const f32x4 uu = b * (vv - ks);
            s_u[tid] = uu;
            Elem<TO>::st4(o + nh * DV + 4 * cb, qs + uu * kqt);
        }
        __syncthreads();
        u = s_u[cb];
    } else {
        __shared__ f32x4 s_pk[Sh::RP][Sh::CB], s_pq[Sh::RP][Sh::CB];
        __shared__ float s_kq[Sh::RP];
        s_pk[r0][cb] = pk;
        s_pq[r0][cb] = pq;
        if (cb == 0) s_kq[r0] = kq;
        __syncthreads();
        f32x4 ks = {0.f, 0.f, 0.f, 0.f}, qs = {0.f, 0.f, 0.f, 0.f};
        float kqt = 0.f;
#pragma unroll
        for (int r = 0; r < Sh::RP; ++r) {
            ks += s_pk[r][cb];
            qs += s_pq[r][cb];
            kqt += s_kq[r];
        }
        u = b * (vv - ks);
        if (r0 == 0) Elem<TO>::st4(o + nh * DV + 4 * cb, qs + u * kqt);
    }

    // 5. rank-1 write
#pragma unroll
    for (int p = 0; p < Sh::R; ++p) {
        const int i = r0 + p * Sh::RP;
        const float ki = s_k[i];
        __builtin_nontemporal_store(s[p] + ki * u,
                                    reinterpret_cast<f32x4 *>(Sh_ + i * DV + 4 * cb));
    }
}

template <typename TI, typename TO, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs &a)
{
    using Sh = DecodeShape<DK, DV>;
    const int64_t heads = (int64_t)a.N * a.H;
    if (heads == 0) return hipSuccess;
    if (heads * Sh::NT >= ((int64_t)1 << 32)) return hipErrorInvalidValue;  // grid size limit
    hipLaunchKernelGGL((kda_decode_kernel<TI, TO, DK, DV>), dim3((unsigned)heads),
                       dim3(Sh::NT), 0, (hipStream_t)a.stream,
                       (const TI *)a.q, (const TI *)a.k, (const TI *)a.v, a.g, a.beta,
                       a.S, (TO *)a.o);
    return hipGetLastError();
}

template <typename TI, typename TO>
static hipError_t dispatch_dims(const DecodeArgs &a)
{
#define KDA_DEC_CASE(DK_, DV_) \
    if (a.d_k == DK_ && a.d_v == DV_) return launch_decode_t<TI, TO, DK_, DV_>(a);
    KDA_DEC_CASE(16, 16) KDA_DEC_CASE(16, 32) KDA_DEC_CASE(16, 64) KDA_DEC_CASE(16, 128)
    KDA_DEC_CASE(32, 16) KDA_DEC_CASE(32, 32) KDA_DEC_CASE(32, 64) KDA_DEC_CASE(32, 128)
    KDA_DEC_CASE(64, 16) KDA_DEC_CASE(64, 32) KDA_DEC_CASE(64, 64) KDA_DEC_CASE(64, 128)
    KDA_DEC_CASE(128, 16) KDA_DEC_CASE(128, 32) KDA_DEC_CASE(128, 64) KDA_DEC_CASE(128, 128)
#undef KDA_DEC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs &a)
{
    if (a.in_bf16) {
        return a.out_bf16 ? dispatch_dims<bf16, bf16>(a) : dispatch_dims<bf16, float>(a);
    }
    return dispatch_dims<float, float>(a);
}

}  // namespace kda
