// KDA chunked backward: gradients of the prefill with respect to q, k, v, g,
// beta and S0, given the cotangents dO of o and dS_T of the final state.
//
// The forward chunk algebra (16-token chunks, every factor referenced to
// the chunk end; the same as the prefill kernel's) is
//     Sd = Diag(gamma) S,  X = V - KE Sd,  U = T X,  O = QE Sd + P U,
//     S' = Sd + Kd^T U,    T = (I + A)^-1 Diag(beta),
//     A = strict_lower(Diag(beta) KE Kd^T),  P = lower_incl(QE Kd^T),
// with gamma = e^{Gc_16}, KE = k E, QE = q E, Kd = k / E, E_r = e^{Gc_r - Gc_16}
// (the state-update equation of the Kimi K3 architecture walkthrough,
// mhpq.cn/news/56770, "KDA 到底在算什么", evaluated 16 tokens at a time).
// Reverse-mode through it, with L the cotangent of S' (the chunk's exit
// state):
//     dU  = P^T dO + Kd L           dX  = T^T dU            dV = dX
//     dSd = QE^T dO + L - KE^T dX    L_prev = Diag(gamma) dSd
//     dQE = dO Sd^T + dP Kd         dP  = lower_incl(dO U^T)
//     dKE = -dX Sd^T + (Diag(beta) dA) Kd
//     dKd = U L^T + dP^T QE + (Diag(beta) dA)^T KE
//     dT  = dU X^T,  dM = dT Diag(beta),  dA = strict_lower(-M^T dM M^T)
//     dbeta_i = sum_r dT[r][i] M[r][i] + sum_s dA[i][s] (KE Kd^T)[i][s]
//     dgamma_i = sum_j dSd[i][j] S[i][j]
// and through the referencing: dq = dQE E, dk = dKE E + dKd / E, the log
// terms dx = dQE QE + dKE KE - dKd Kd of Gc_r - Gc_16, dgamma gamma of
// Gc_16, and a reverse cumulative sum over the chunk for dg.
//
// The carried cotangent L only meets products that contract over d_k or
// over the 16 tokens, so its columns split into blocks as the forward's
// state does; the products that contract over d_v (dO Sd^T, dX Sd^T,
// U L^T, dU X^T, dO U^T, dgamma) only feed the per-chunk gradients.  Two
// implementations:
//
//  * bf16 inputs, d_k >= 32 (the matrix-core path, second half of this
//    file): kda_bwd_sweep_mfma carries L through the chunks in reverse and
//    writes dv, dS0 and every chunk's exit cotangent; kda_bwd_chunk then
//    forms all of a chunk's remaining gradients from its checkpointed
//    entry state (stored by the checkpointing forward as the decayed Sd in
//    bf16 hi/lo operand form) and exit cotangent, every (chunk, head) in
//    parallel.
//  * fp32 inputs (the precision reference) and d_k = 16 (first half):
//    kda_bwd_sweep runs one workgroup per (sequence, head, block of
//    columns) backwards over the chunks and writes dv, dS0 and per-block
//    partial sums of the d_v-contracted products; kda_bwd_finish, one
//    workgroup per (chunk, head), adds them up and forms dq, dk, dg and
//    dbeta.  Arithmetic is fp32 on the vector ALU (LDS-staged products,
//    each thread accumulating a small tile of outputs).
#include <cstddef>

#include "kda_chunk.h"
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace bwd {

constexpr int NT = 512;            // threads of both kernels
constexpr int C = 16;              // chunk = decay tile

// floats per (chunk slot, head, column block) of the partial sums
template <int DK>
struct Part {
    static constexpr int QE = 0, KE = C * DK, KD = 2 * C * DK, T = 3 * C * DK;
    static constexpr int P = T + C * C, GAM = P + C * C;
    static constexpr int SIZE = GAM + DK;
};

// C[m][n] (m < M, n < N) over tiles of TM x TN per thread: acc = sum_k
// a(m, k) b(k, n); store(m, n, acc) once per output
template <int TM, int TN, typename FA, typename FB, typename FS>
__device__ __forceinline__ void tile_gemm(int M, int N, int K, FA a, FB b, FS store)
{
    const int tn = N / TN, tiles = (M / TM) * tn;
    for (int e = threadIdx.x; e < tiles; e += NT) {
        const int m0 = (e / tn) * TM, n0 = (e % tn) * TN;
        float acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;
        for (int kk = 0; kk < K; ++kk) {
            float av[TM], bv[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) av[i] = a(m0 + i, kk);
#pragma unroll
            for (int j = 0; j < TN; ++j) bv[j] = b(kk, n0 + j);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) store(m0 + i, n0 + j, acc[i][j]);
    }
}

// Chunk operands shared by both kernels: cumulative log2-decay, E, 1/E,
// gamma, QE, KE, Kd, KE gamma, A, M = (I + A)^-1, T, P, beta.
template <int DK>
struct Ops {
    float G[C][DK + 1];                // Gc_r - Gc_16 (log2), then reused
    float QE[C][DK + 1], KE[C][DK + 1], KD[C][DK + 1], KG[C][DK + 1];
    float gam[DK];
    float A[C][C + 1], M[C][C + 1], T[C][C + 1], P[C][C + 1], KK[C][C + 1];
    float beta[C];
};

template <typename TI>
__device__ __forceinline__ float ldx(const TI *p) { return Elem<TI>::ld(p); }

// load one chunk (tokens tok0 .. tok0 + n - 1 of head h) and form its
// operands; n <= 16, padded tokens are the identity (k = q = 0, g = 0,
// beta = 0)
template <typename TI, int DK>
__device__ void chunk_ops(Ops<DK> &o, const TI *q, const TI *k, const float *g,
                          const float *beta, int64_t tok0, int n, int H, int h)
{
    const int tid = threadIdx.x;
    // cumulative log2-decay per channel (one thread per channel)
    for (int c = tid; c < DK; c += NT) {
        float s = 0.f;
        for (int r = 0; r < C; ++r) {
            const float gr = r < n ? g[((tok0 + r) * H + h) * DK + c] : 0.f;
            s = __builtin_fmaf(gr, LOG2E, s);
            o.G[r][c] = s;
        }
        for (int r = 0; r < C; ++r) o.G[r][c] -= s;
        o.gam[c] = fast_exp2(s);
    }
    if (tid < C) o.beta[tid] = tid < n ? beta[(tok0 + tid) * H + h] : 0.f;
    __syncthreads();
    for (int e = tid; e < C * DK; e += NT) {
        const int r = e / DK, c = e % DK;
        const int64_t off = ((tok0 + r) * H + h) * DK + c;
        const float qv = r < n ? ldx(q + off) : 0.f, kv = r < n ? ldx(k + off) : 0.f;
        const float x = o.G[r][c];                   // (Gc_r - Gc_16) log2(e) >= 0
        const float E = fast_exp2(x), F = fast_exp2(-x);
        o.QE[r][c] = qv * E;
        o.KE[r][c] = kv * E;
        o.KD[r][c] = kv * F;
        o.KG[r][c] = kv * E * o.gam[c];
    }
    __syncthreads();
    // KK = KE Kd^T and P = lower_incl(QE Kd^T), 16 x 16 each
    tile_gemm<1, 1>(C, C, DK, [&](int m, int kk) { return o.KE[m][kk]; },
                    [&](int kk, int nn) { return o.KD[nn][kk]; },
                    [&](int m, int nn, float v) { o.KK[m][nn] = v; });
    tile_gemm<1, 1>(C, C, DK, [&](int m, int kk) { return o.QE[m][kk]; },
                    [&](int kk, int nn) { return o.KD[nn][kk]; },
                    [&](int m, int nn, float v) { o.P[m][nn] = nn <= m ? v : 0.f; });
    __syncthreads();
    for (int e = tid; e < C * C; e += NT) {
        const int r = e / C, i = e % C;
        o.A[r][i] = i < r ? o.beta[r] * o.KK[r][i] : 0.f;
    }
    __syncthreads();
    // M = (I + A)^-1 by forward substitution, one column per thread
    if (tid < C) {
        const int j = tid;
        for (int r = 0; r < C; ++r) {
            float x = r == j ? 1.f : 0.f;
            for (int i = 0; i < r; ++i) x = __builtin_fmaf(-o.A[r][i], o.M[i][j], x);
            o.M[r][j] = x;
        }
    }
    __syncthreads();
    for (int e = tid; e < C * C; e += NT) {
        const int r = e / C, i = e % C;
        o.T[r][i] = o.M[r][i] * o.beta[i];
    }
    __syncthreads();
}

template <int DK, int BV>
struct SweepSmem {
    Ops<DK> o;
    float S[DK][BV + 1];               // chunk-entry state (this column block)
    float L[DK][BV + 1];               // cotangent of the chunk-exit state
    float V[C][BV + 1], DO[C][BV + 1], X[C][BV + 1], U[C][BV + 1], DU[C][BV + 1],
        DX[C][BV + 1];
};

}  // namespace bwd

// One workgroup per (sequence n, head h, column block); chunks in reverse.
template <typename TI, int DK, int DV, int BV>
__global__ __launch_bounds__(bwd::NT)
void kda_bwd_sweep(const TI *__restrict__ q, const TI *__restrict__ k,
                   const TI *__restrict__ v, const float *__restrict__ g,
                   const float *__restrict__ beta, const TI *__restrict__ dO,
                   const float *__restrict__ dST, const int32_t *__restrict__ cu_seqlens,
                   int32_t seqlen, int32_t n_tokens, int32_t H, const float *__restrict__ ckpt,
                   float *__restrict__ part, float *__restrict__ dv, float *__restrict__ dS0)
{
    using namespace bwd;
    constexpr int NB = DV / BV;
    __shared__ SweepSmem<DK, BV> sm;
    const int tid = threadIdx.x;
    const int blk = blockIdx.x % NB;
    const int chain = blockIdx.x / NB;          // n * H + h
    const int n = chain / H, h = chain % H;
    const int col0 = blk * BV;
    int64_t bos, T;
    if (cu_seqlens) {
        const int32_t c0 = cu_seqlens[n], c1 = cu_seqlens[n + 1];
        const int32_t a0 = c0 < 0 ? 0 : (c0 > n_tokens ? n_tokens : c0);
        const int32_t a1 = c1 < 0 ? 0 : (c1 > n_tokens ? n_tokens : c1);
        bos = a0;
        T = a1 > a0 ? a1 - a0 : 0;
    } else {
        bos = (int64_t)n * seqlen;
        T = seqlen;
    }
    const int nch = (int)((T + C - 1) / C);
    const int64_t slot0 = bos / C + n;
    // L = dS_T (or 0)
    for (int e = tid; e < DK * BV; e += NT) {
        const int i = e / BV, j = e % BV;
        sm.L[i][j] = dST ? dST[(int64_t)chain * DK * DV + i * DV + col0 + j] : 0.f;
    }
    for (int c = nch - 1; c >= 0; --c) {
        const int64_t tok0 = bos + (int64_t)c * C;
        const int nt = (int)(T - (int64_t)c * C < C ? T - (int64_t)c * C : C);
        __syncthreads();
        chunk_ops<TI, DK>(sm.o, q, k, g, beta, tok0, nt, H, h);
        // the checkpoint's 16 x 16 tiles: element (row i, column c) of tile
        // (c / 16, i / 16) sits at lane (c % 16) + 16 ((i % 16) / 4), word i % 4
        const float *ck = ckpt + ((slot0 + c) * H + h) * (int64_t)(DK * DV);
        for (int e = tid; e < DK * BV; e += NT) {
            const int i = e / BV, j = e % BV, cc = col0 + j;
            sm.S[i][j] = ck[(((cc / 16) * (DK / 16) + i / 16) * WAVE + (cc % 16) +
                            16 * ((i % 16) / 4)) * 4 + i % 4];
        }
        for (int e = tid; e < C * BV; e += NT) {
            const int r = e / BV, j = e % BV;
            const int64_t off = ((tok0 + r) * H + h) * DV + col0 + j;
            sm.V[r][j] = r < nt ? ldx(v + off) : 0.f;
            sm.DO[r][j] = r < nt ? ldx(dO + off) : 0.f;
        }
        __syncthreads();
        // X = V - (KE gamma) S;  dU (first part) = P^T dO + Kd L
        tile_gemm<2, 2>(C, BV, DK, [&](int m, int kk) { return sm.o.KG[m][kk]; },
                        [&](int kk, int nn) { return sm.S[kk][nn]; },
                        [&](int m, int nn, float x) { sm.X[m][nn] = sm.V[m][nn] - x; });
        tile_gemm<2, 2>(C, BV, DK, [&](int m, int kk) { return sm.o.KD[m][kk]; },
                        [&](int kk, int nn) { return sm.L[kk][nn]; },
                        [&](int m, int nn, float x) { sm.DU[m][nn] = x; });
        __syncthreads();
        // U = T X;  dU += P^T dO
        tile_gemm<2, 2>(C, BV, C, [&](int m, int kk) { return sm.o.T[m][kk]; },
                        [&](int kk, int nn) { return sm.X[kk][nn]; },
                        [&](int m, int nn, float x) { sm.U[m][nn] = x; });
        tile_gemm<2, 2>(C, BV, C, [&](int m, int kk) { return sm.o.P[kk][m]; },
                        [&](int kk, int nn) { return sm.DO[kk][nn]; },
                        [&](int m, int nn, float x) { sm.DU[m][nn] += x; });
        __syncthreads();
        // dX = T^T dU (= dV, written out); partial dKd = U L^T (L still the
        // exit cotangent); partial dT = dU X^T, dP = dO U^T
        float *pp = part + (((slot0 + c) * H + h) * NB + blk) * (int64_t)Part<DK>::SIZE;
        tile_gemm<2, 2>(C, BV, C, [&](int m, int kk) { return sm.o.T[kk][m]; },
                        [&](int kk, int nn) { return sm.DU[kk][nn]; },
                        [&](int m, int nn, float x) {
                            sm.DX[m][nn] = x;
                            if (m < nt) dv[((tok0 + m) * H + h) * DV + col0 + nn] = x;
                        });
        __syncthreads();
        tile_gemm<2, 4>(C, DK, BV, [&](int m, int kk) { return sm.U[m][kk]; },
                        [&](int kk, int nn) { return sm.L[nn][kk]; },
                        [&](int m, int nn, float x) { pp[Part<DK>::KD + m * DK + nn] = x; });
        tile_gemm<1, 1>(C, C, BV, [&](int m, int kk) { return sm.DU[m][kk]; },
                        [&](int kk, int nn) { return sm.X[nn][kk]; },
                        [&](int m, int nn, float x) { pp[Part<DK>::T + m * C + nn] = x; });
        tile_gemm<1, 1>(C, C, BV, [&](int m, int kk) { return sm.DO[m][kk]; },
                        [&](int kk, int nn) { return sm.U[nn][kk]; },
                        [&](int m, int nn, float x) { pp[Part<DK>::P + m * C + nn] = x; });
        // partial dQE = dO Sd^T, dKE = -dX Sd^T (Sd = gamma S)
        tile_gemm<2, 4>(C, DK, BV, [&](int m, int kk) { return sm.DO[m][kk]; },
                        [&](int kk, int nn) { return sm.S[nn][kk]; },
                        [&](int m, int nn, float x) {
                            pp[Part<DK>::QE + m * DK + nn] = x * sm.o.gam[nn];
                        });
        tile_gemm<2, 4>(C, DK, BV, [&](int m, int kk) { return sm.DX[m][kk]; },
                        [&](int kk, int nn) { return sm.S[nn][kk]; },
                        [&](int m, int nn, float x) {
                            pp[Part<DK>::KE + m * DK + nn] = -x * sm.o.gam[nn];
                        });
        __syncthreads();
        // dSd = QE^T dO + L - KE^T dX; partial dgamma_i = sum_j dSd S; then
        // L <- Diag(gamma) dSd, in place (every read of the old L is done)
        tile_gemm<2, 2>(DK, BV, C, [&](int m, int kk) { return sm.o.QE[kk][m]; },
                        [&](int kk, int nn) { return sm.DO[kk][nn]; },
                        [&](int m, int nn, float x) { sm.L[m][nn] += x; });
        __syncthreads();
        tile_gemm<2, 2>(DK, BV, C, [&](int m, int kk) { return sm.o.KE[kk][m]; },
                        [&](int kk, int nn) { return sm.DX[kk][nn]; },
                        [&](int m, int nn, float x) { sm.L[m][nn] -= x; });
        __syncthreads();
        for (int i = tid; i < DK; i += NT) {
            float s = 0.f;
            for (int j = 0; j < BV; ++j) s = __builtin_fmaf(sm.L[i][j], sm.S[i][j], s);
            pp[Part<DK>::GAM + i] = s;
        }
        __syncthreads();
        for (int e = tid; e < DK * BV; e += NT) {
            const int i = e / BV, j = e % BV;
            sm.L[i][j] *= sm.o.gam[i];
        }
    }
    __syncthreads();
    if (dS0) {
        for (int e = tid; e < DK * BV; e += NT) {
            const int i = e / BV, j = e % BV;
            dS0[(int64_t)chain * DK * DV + i * DV + col0 + j] = sm.L[i][j];
        }
    }
}

namespace bwd {
template <int DK>
struct FinishSmem {
    Ops<DK> o;
    float dQE[C][DK + 1], dKE[C][DK + 1], dKD[C][DK + 1], dX[C][DK + 1];
    float dT[C][C + 1], dP[C][C + 1], dM[C][C + 1], W[C][C + 1], dA[C][C + 1];
    float dgam[DK];
    float db[C];
};
}  // namespace bwd

// One workgroup per (chunk slot, head): sum the blocks' partials and form
// dq, dk, dg, dbeta of the chunk's tokens.  Chunk c of sequence n has slot
// bos_n / 16 + n + c; these starts grow with n, so a slot's sequence is
// found by binary search (slots between sequences exit at once).
template <typename TI, int DK, int NB>
__global__ __launch_bounds__(bwd::NT)
void kda_bwd_finish(const TI *__restrict__ q, const TI *__restrict__ k,
                    const float *__restrict__ g, const float *__restrict__ beta,
                    const int32_t *__restrict__ cu_seqlens, int32_t n_seqs, int32_t seqlen,
                    int32_t n_tokens, int32_t H, const float *__restrict__ part,
                    float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dg,
                    float *__restrict__ db)
{
    using namespace bwd;
    __shared__ FinishSmem<DK> sm;
    const int tid = threadIdx.x;
    const int64_t slot = blockIdx.x / H;
    const int h = blockIdx.x % H;
    auto bos_of = [&](int s) -> int64_t {
        if (!cu_seqlens) return (int64_t)s * seqlen;
        const int32_t c0 = cu_seqlens[s];
        return c0 < 0 ? 0 : (c0 > n_tokens ? n_tokens : c0);
    };
    // largest n with bos_n / 16 + n <= slot
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (bos_of(mid) / C + mid <= slot) lo = mid;
        else hi = mid - 1;
    }
    const int n = lo;
    const int64_t bos = bos_of(n);
    int64_t T;
    if (cu_seqlens) {
        const int32_t c1 = cu_seqlens[n + 1];
        const int64_t a1 = c1 < 0 ? 0 : (c1 > n_tokens ? n_tokens : c1);
        T = a1 > bos ? a1 - bos : 0;
    } else {
        T = seqlen;
    }
    const int64_t c = slot - (bos / C + n);
    if (c < 0 || c * C >= T) return;
    const int64_t tok0 = bos + (int64_t)c * C;
    const int nt = (int)(T - (int64_t)c * C < C ? T - (int64_t)c * C : C);
    chunk_ops<TI, DK>(sm.o, q, k, g, beta, tok0, nt, H, h);
    // sum the column blocks' partials
    const float *pp = part + ((slot * H + h) * NB) * (int64_t)Part<DK>::SIZE;
    for (int e = tid; e < C * DK; e += NT) {
        const int r = e / DK, i = e % DK;
        float a = 0.f, b = 0.f, d = 0.f;
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) {
            const float *p = pp + bl * Part<DK>::SIZE;
            a += p[Part<DK>::QE + e];
            b += p[Part<DK>::KE + e];
            d += p[Part<DK>::KD + e];
        }
        sm.dQE[r][i] = a;
        sm.dKE[r][i] = b;
        sm.dKD[r][i] = d;
    }
    for (int e = tid; e < C * C; e += NT) {
        const int r = e / C, i = e % C;
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) {
            a += pp[bl * Part<DK>::SIZE + Part<DK>::T + e];
            b += pp[bl * Part<DK>::SIZE + Part<DK>::P + e];
        }
        sm.dT[r][i] = a;
        sm.dP[r][i] = i <= r ? b : 0.f;          // P is lower triangular incl.
    }
    for (int i = tid; i < DK; i += NT) {
        float a = 0.f;
#pragma unroll
        for (int bl = 0; bl < NB; ++bl) a += pp[bl * Part<DK>::SIZE + Part<DK>::GAM + i];
        sm.dgam[i] = a;
    }
    __syncthreads();
    // T = M Diag(beta): dM = dT Diag(beta), dbeta_i = sum_r dT[r][i] M[r][i]
    for (int e = tid; e < C * C; e += NT) {
        const int r = e / C, i = e % C;
        sm.dM[r][i] = sm.dT[r][i] * sm.o.beta[i];
    }
    if (tid < C) {
        float s = 0.f;
        for (int r = 0; r < C; ++r) s = __builtin_fmaf(sm.dT[r][tid], sm.o.M[r][tid], s);
        sm.db[tid] = s;
    }
    __syncthreads();
    // dA = strict_lower(-M^T dM M^T): W = M^T dM, then dA = -W M^T
    tile_gemm<1, 1>(C, C, C, [&](int m, int kk) { return sm.o.M[kk][m]; },
                    [&](int kk, int nn) { return sm.dM[kk][nn]; },
                    [&](int m, int nn, float x) { sm.W[m][nn] = x; });
    __syncthreads();
    tile_gemm<1, 1>(C, C, C, [&](int m, int kk) { return sm.W[m][kk]; },
                    [&](int kk, int nn) { return sm.o.M[nn][kk]; },
                    [&](int m, int nn, float x) { sm.dA[m][nn] = nn < m ? -x : 0.f; });
    __syncthreads();
    // A = Diag(beta) KK (strict lower): dbeta_r += sum_s dA[r][s] KK[r][s];
    // the product's cotangent is Diag(beta) dA, kept in dA
    if (tid < C) {
        float s = 0.f;
        for (int i = 0; i < C; ++i) s = __builtin_fmaf(sm.dA[tid][i], sm.o.KK[tid][i], s);
        sm.db[tid] += s;
    }
    __syncthreads();
    for (int e = tid; e < C * C; e += NT) {
        const int r = e / C, i = e % C;
        sm.dA[r][i] *= sm.o.beta[r];
    }
    __syncthreads();
    // dQE += dP Kd;  dKE += dA Kd;  dKd += dP^T QE + dA^T KE
    tile_gemm<1, 4>(C, DK, C, [&](int m, int kk) { return sm.dP[m][kk]; },
                    [&](int kk, int nn) { return sm.o.KD[kk][nn]; },
                    [&](int m, int nn, float x) { sm.dQE[m][nn] += x; });
    tile_gemm<1, 4>(C, DK, C, [&](int m, int kk) { return sm.dA[m][kk]; },
                    [&](int kk, int nn) { return sm.o.KD[kk][nn]; },
                    [&](int m, int nn, float x) { sm.dKE[m][nn] += x; });
    tile_gemm<1, 4>(C, DK, C, [&](int m, int kk) { return sm.dP[kk][m]; },
                    [&](int kk, int nn) { return sm.o.QE[kk][nn]; },
                    [&](int m, int nn, float x) { sm.dKD[m][nn] += x; });
    __syncthreads();
    tile_gemm<1, 4>(C, DK, C, [&](int m, int kk) { return sm.dA[kk][m]; },
                    [&](int kk, int nn) { return sm.o.KE[kk][nn]; },
                    [&](int m, int nn, float x) { sm.dKD[m][nn] += x; });
    __syncthreads();
    // through E = e^{x}, 1/E: dq, dk, and the log terms dx of x = Gc_r - Gc_16
    for (int e = tid; e < C * DK; e += NT) {
        const int r = e / DK, i = e % DK;
        const float x = sm.o.G[r][i];                 // log2 units
        const float E = fast_exp2(x), F = fast_exp2(-x);
        const float dqe = sm.dQE[r][i], dke = sm.dKE[r][i], dkd = sm.dKD[r][i];
        if (r < nt) {
            const int64_t off = ((tok0 + r) * H + h) * DK + i;
            dq[off] = dqe * E;
            dk[off] = dke * E + dkd * F;
        }
        sm.dX[r][i] = dqe * sm.o.QE[r][i] + dke * sm.o.KE[r][i] - dkd * sm.o.KD[r][i];
    }
    __syncthreads();
    // dGc_r = dx_r (r < 15); dGc_16 gets -sum_r dx_r + dgamma gamma; then
    // dg_s = sum_{r >= s} dGc_r over the chunk
    for (int i = tid; i < DK; i += NT) {
        float tot = 0.f;
        for (int r = 0; r < C; ++r) tot += sm.dX[r][i];
        float acc = sm.dgam[i] * sm.o.gam[i] - tot + sm.dX[C - 1][i];
        for (int r = C - 1; r >= 0; --r) {
            if (r < C - 1) acc += sm.dX[r][i];
            if (r < nt) dg[((tok0 + r) * H + h) * DK + i] = acc;
        }
    }
    if (tid < nt) db[(tok0 + tid) * H + h] = sm.db[tid];
}

// ===========================================================================
// Matrix-core backward (bf16 inputs, d_k >= 32)
//
// The carried cotangent runs the chain
//     dU = P^T dO + Kd L,   dX = T^T dU,   L <- Diag(gamma) (L + QE^T dO - KE^T dX)
// which has the shape of the forward's state chain (a 16 x d_k by d_k x BV
// product, a 16-token triangular product, a rank-16 update of the carried
// d_k x BV block), so kda_bwd_sweep_mfma keeps the forward kernel's
// organisation: per (sequence, head, block of BV columns) one workgroup,
// consumer waves holding L in the accumulator layout, builder waves forming
// the operands of chunk c + 2 in a three-slot LDS ring (now in reverse chunk
// order and with dO in place of v; with d_k = 128 and four consumers two
// auxiliary waves move the dO block, as they move v in the forward), two
// helper waves forming T^T and P^T of chunk c + 1.  Per chunk it writes
// dV = dX and the exit cotangent L of the chunk (in the 16 x 16 tiles of the
// state checkpoints); after chunk 0, dS0.
//
// kda_bwd_chunk then takes every (chunk, head) independently: from the
// chunk-start state (checkpointed as the decayed Sd in bf16 hi/lo operand
// form) and the exit cotangent L it re-forms X, U, dU and dX
// one block of 16 value columns at a time and accumulates the products that
// contract over the value columns (dO Sd^T, dX Sd^T, L U^T, dU X^T, dO U^T
// and the row sums of L o Sd) on the matrix cores; the rest is 16 x 16 and
// 16 x d_k algebra.  Tiles whose contraction runs along the value columns
// are transposed on the matrix core (a product with the identity on one
// half of the K slots, separately for the hi and the lo part).
// ===========================================================================
namespace bwdm {

template <int DK, int NW>
using SC = Cfg<bf16, DK, NW, 3, false, MODE_SWEEP>;
template <int DK>
using CC = Cfg<bf16, DK, 1, 3, false, MODE_CHUNK>;

struct SweepParams {
    const bf16 *q, *k, *dO;
    const float *g, *beta, *dST;
    const int32_t *cu_seqlens;
    int32_t seqlen, n_tokens, n_chains, chains8, H;
    float *Lck, *dv, *dS0;
};

__device__ __forceinline__ bf16x4 lo4(bf16x8 x) { return __builtin_shufflevector(x, x, 0, 1, 2, 3); }
__device__ __forceinline__ bf16x4 hi4(bf16x8 x) { return __builtin_shufflevector(x, x, 4, 5, 6, 7); }

// B operand of the identity on one half of the K slots: slot 8 kg + i
// (i < 4 for half 0, i >= 4 for half 1) stands for row 4 kg + i % 4 and the
// other half is zero, so a product of a 4 + 4 slot operand (as the A
// operand) with it is the transposed tile of that half, exact in fp32
__device__ __forceinline__ bf16x8 eye_half(int lane, int half)
{
    const int n = lane & 15, kg = lane >> 4;
    bf16x8 e;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        e[i] = ((i >> 2) == half && 4 * kg + (i & 3) == n) ? (bf16)1.0f : (bf16)0.0f;
    return e;
}
// four exact bf16 values held in fp32
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x)
{
    return __builtin_bit_cast(bf16x4, u32x2{pack2(x[0], x[1]), pack2(x[2], x[3])});
}

// operands of chunk c + 1 that its builders have finished, read before the
// barrier that ends chunk c
struct AheadB {
    bf16x4 v;            // dO of the lane's column, tokens 4 g4 .. 4 g4 + 3
    bf16x8 dh, dl;       // Kd hi / lo, first 32-deep step
};
template <class C>
__device__ __forceinline__ void read_ahead_b(const Buf<C> &B, AheadB &a, int wave, int lane)
{
    const int j = lane & 15, g4 = lane >> 4;
    a.v = ld4b(&B.VT[16 * wave + j][4 * g4]);
    a.dh = ld8b(&B.DH[j][8 * g4]);
    a.dl = ld8b(&B.DL[j][8 * g4]);
}

// one chunk of the cotangent chain for this wave's 16 columns; L holds rows
// 16 t + 4 g4 + i of column j (lane (j, g4)); returns dX (lane (j, g4):
// tokens 4 g4 + i of column j)
template <class C>
__device__ __forceinline__ f32x4 consume_sweep(const Buf<C> &B, f32x4 (&L)[C::DK / 16],
                                               const AheadB &ah, int lane)
{
    constexpr int NS = C::DK / 32;
    const int j = lane & 15, g4 = lane >> 4;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const NegEye ne = neg_eye(lane);
    const bf16x8 dov = cat(ah.v, ah.v);
    // T^T and P^T of the chunk are final when the chunk starts
    const bf16x8 pt = ld8b(&B.PH[j][8 * g4]);
    const bf16x8 tth = ld8b(&B.TH[j][8 * g4]), ttl = ld8b(&B.TL[j][8 * g4]);
    // dU = P^T dO + Kd L: [PTh | PTl] against [dO | dO]; Kd (hi, lo) against
    // L as a hi/lo pair, K slots in the stored channel order of Kd
    f32x4 du = mma32(pt, dov, zero);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        bf16x8 lh, ll;
        split8(L[2 * s], L[2 * s + 1], ne, lh, ll);
        const int kk = 32 * s + 8 * g4;
        const bf16x8 dh = s == 0 ? ah.dh : ld8b(&B.DH[j][kk]);
        const bf16x8 dl = s == 0 ? ah.dl : ld8b(&B.DL[j][kk]);
        du = mma32(dh, lh, du);
        du = mma32(dl, lh, du);
        du = mma32(dh, ll, du);
    }
    // L += QE^T dO (every read of the old L went into the splits above)
#pragma unroll
    for (int t = 0; t < C::DK / 16; ++t)
        L[t] = mma32(ld8b(&B.KQ[16 * t + j][32 + 8 * g4]), dov, L[t]);
    // dX = T^T dU: [TTh | TTh] and [TTl | TTl] against [dUh; dUl]
    bf16x4 uh, ul;
    split4(du, ne, uh, ul);
    const bf16x8 duhl = cat(uh, ul);
    f32x4 dx = mma32(tth, duhl, zero);
    dx = mma32(ttl, duhl, dx);
    // L += -KE^T dX, then the chunk's decay: L_prev = Diag(gamma) dSd
    bf16x4 xh, xl;
    split4(dx, ne, xh, xl);
    const bf16x8 bxh = cat(xh, xh), bxl = cat(xl, xl);
#pragma unroll
    for (int t = 0; t < C::DK / 16; ++t) {
        const bf16x8 a = ld8b(&B.KQ[16 * t + j][8 * g4]);
        L[t] = mma32(a, bxh, L[t]);
        L[t] = mma32(a, bxl, L[t]);
        L[t] *= *reinterpret_cast<const f32x4 *>(&B.DEC[16 * t + 4 * g4]);
    }
    return dx;
}

}  // namespace bwdm

// One workgroup per (sequence, head, block of BV columns); chunks in reverse.
template <int DK, int DV, int NW>
__global__ __launch_bounds__((bwdm::SC<DK, NW>::NT), 1)
void kda_bwd_sweep_mfma(const bwdm::SweepParams p)
{
    using namespace bwdm;
    using C = SC<DK, NW>;
    constexpr int NB = DV / C::BV;
    __shared__ Smem<C> sm;
    const int H = p.H;
    // workgroup -> job as in the prefill: the blocks of a chain share an XCD
    const int bid = blockIdx.x;
    const int xcd = bid & 7, rest = bid >> 3;
    const int vb = rest % NB;
    const int chain = (rest / NB) * 8 + xcd;
    if (chain >= p.n_chains) return;
    const int h = chain % H;
    int n = chain / H;
    if (p.cu_seqlens && p.n_chains / H <= kLptMaxSeqs)
        n = __builtin_amdgcn_readfirstlane(
            seq_of_rank(p.cu_seqlens, p.n_chains / H, n, threadIdx.x & 63));
    const int64_t state_of = (int64_t)n * H + h;
    int64_t bos, T;
    if (p.cu_seqlens) {
        const int32_t c0 = p.cu_seqlens[n], c1 = p.cu_seqlens[n + 1];
        const int32_t a0 = c0 < 0 ? 0 : (c0 > p.n_tokens ? p.n_tokens : c0);
        const int32_t a1 = c1 < 0 ? 0 : (c1 > p.n_tokens ? p.n_tokens : c1);
        bos = a0;
        T = a1 > a0 ? a1 - a0 : 0;
    } else {
        bos = (int64_t)n * p.seqlen;
        T = p.seqlen;
    }
    const int col_base = vb * C::BV;
    bos = uniform64(bos);
    const int Tn = __builtin_amdgcn_readfirstlane((int)T);
    const int nch = (Tn + 15) / 16;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_cons = wave < NW;
    const bool is_build = !is_cons && wave < NW + C::NBW;
    const bool is_aux = C::AUX && wave >= NW + C::NBW + 2;
    const int bw = wave - NW, btid = tid - C::NC;
    const int j = lane & 15, g4 = lane >> 4;

    auto ntok_of = [&](int rc) -> int {
        const int rem = Tn - 16 * rc;
        return rem < 0 ? 0 : (rem < 16 ? rem : 16);
    };
    // processing step cc takes chunk nch - 1 - cc; steps past the last
    // chunk read nothing
    auto chunk_of = [&](int cc) -> int { return cc < nch ? nch - 1 - cc : 0; };
    auto ntok_step = [&](int cc) -> int { return cc < nch ? ntok_of(nch - 1 - cc) : 0; };
    auto slot = [&](int s) -> Buf<C> & { return sm.buf[__builtin_amdgcn_readfirstlane(s)]; };

    // the phase plan of the prefill kernel, over processing steps
    if (is_build) {
        constexpr int NR = C::NR;
        Raw<C> r[NR];
        auto load = [&](Raw<C> &x, int cc) {
            load_raw<C>(x, p.q, p.k, p.dO, p.g, p.beta, bos + 16 * (int64_t)chunk_of(cc),
                        ntok_step(cc), ntok_step(cc), H, h, DV, col_base, bw, lane, btid);
        };
#pragma unroll
        for (int i = 0; i < NR; ++i) load(r[i], i);
        if (nch > 0) build<C>(sm.buf[0], r[0], bw, lane, btid, 1.f);
        load(r[0], NR);
        if (nch > 1) build<C>(sm.buf[1], r[1], bw, lane, btid, 1.f);
        load(r[1], NR + 1);
        __syncthreads();
        __syncthreads();
        int c = 0;
#pragma unroll 1
        for (; c + NR <= nch; c += NR) {
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                if (c + i + 2 < nch) build<C>(slot((c + i + 2) % 3), r[(i + 2) % NR], bw, lane, btid, 1.f);
                load(r[(i + 2) % NR], c + i + 2 + NR);
                __syncthreads();
            }
        }
#pragma unroll
        for (int i = 0; i < NR - 1; ++i) {
            if (c + i < nch) {
                if (c + i + 2 < nch) build<C>(slot((c + i + 2) % 3), r[(i + 2) % NR], bw, lane, btid, 1.f);
                __syncthreads();
            }
        }
    } else if (is_aux) {
        if constexpr (C::AUX) {
            // the dO block of step c + 2, on the builders' schedule
            const int a = tid - (NW + C::NBW + 2) * WAVE;
            constexpr int NR = 3;
            AuxV r[NR];
            auto load = [&](int i, int cc) {
                aux_load_v<C>(r[i], p.dO, bos + 16 * (int64_t)chunk_of(cc), ntok_step(cc), H, h,
                              DV, col_base, a);
            };
#pragma unroll
            for (int i = 0; i < NR; ++i) load(i, i);
            if (nch > 0) aux_write_v<C>(sm.buf[0], r[0], a);
            load(0, NR);
            if (nch > 1) aux_write_v<C>(sm.buf[1], r[1], a);
            load(1, NR + 1);
            __syncthreads();
            __syncthreads();
            int c = 0;
#pragma unroll 1
            for (; c + NR <= nch; c += NR) {
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    if (c + i + 2 < nch) aux_write_v<C>(slot((c + i + 2) % 3), r[(i + 2) % NR], a);
                    load((i + 2) % NR, c + i + 2 + NR);
                    __syncthreads();
                }
            }
#pragma unroll
            for (int i = 0; i < NR - 1; ++i) {
                if (c + i < nch) {
                    if (c + i + 2 < nch) aux_write_v<C>(slot((c + i + 2) % 3), r[(i + 2) % NR], a);
                    __syncthreads();
                }
            }
        }
    } else if (!is_cons) {
        auto help = [&](Buf<C> &B) {
            if (wave == NW + C::NBW) helper<C, 0>(B, lane);
            else helper<C, 1>(B, lane);
        };
        __syncthreads();
        if (nch > 0) help(sm.buf[0]);
        __syncthreads();
#pragma unroll 1
        for (int c = 0; c < nch; ++c) {
            if (c + 1 < nch) help(slot((c + 1) % 3));
            __syncthreads();
        }
    } else {
        // L[:, col_base + 16 wave + j], rows 16 t + 4 g4 + i
        f32x4 L[DK / 16];
        const int col = col_base + 16 * wave + j;
#pragma unroll
        for (int t = 0; t < DK / 16; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                L[t][i] = p.dST ? p.dST[state_of * DK * DV + (int64_t)(16 * t + 4 * g4 + i) * DV + col]
                                : 0.f;
        // exit-cotangent tiles of this wave's columns, chunk 0 of the sequence
        f32x4 *lk = reinterpret_cast<f32x4 *>(p.Lck + ((bos / 16 + n) * H + h) * (int64_t)(DK * DV)) +
                    ((col_base / 16 + wave) * (DK / 16)) * WAVE + lane;
        const int drow = H * DV * 4;          // bytes per token of dv (< 2^27, host)
        __syncthreads();
        __syncthreads();
        AheadB ah;
        read_ahead_b<C>(sm.buf[0], ah, wave, lane);
#pragma unroll 1
        for (int cc = 0; cc < nch; ++cc) {
            const int rc = nch - 1 - cc;
#pragma unroll
            for (int t = 0; t < DK / 16; ++t)   // read once, by the chunk kernel: streamed
                __builtin_nontemporal_store(L[t], &lk[(int64_t)rc * H * (DK * DV / 4) + t * WAVE]);
            const f32x4 dx = consume_sweep<C>(slot(cc % 3), L, ah, lane);
            const rsrc_t rd = make_rsrc(p.dv + (bos + 16 * (int64_t)rc) * H * DV, ntok_of(rc) * drow);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                bstore(rd, (4 * g4 + i) * drow + (h * DV + col) * 4, dx[i]);
            read_ahead_b<C>(slot((cc + 1) % 3), ah, wave, lane);
            __syncthreads();
        }
        if (p.dS0) {
#pragma unroll
            for (int t = 0; t < DK / 16; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p.dS0[state_of * DK * DV + (int64_t)(16 * t + 4 * g4 + i) * DV + col] = L[t][i];
        }
    }
}

namespace bwdm {

struct ChunkParams {
    const bf16 *q, *k, *v, *dO;
    const float *g, *beta;
    const int32_t *cu_seqlens;
    int32_t n_seqs, seqlen, n_tokens, H;
    const float *Sck, *Lck;
    float *dq, *dk, *dg, *db;
};

template <int DK, int DV>
struct ChunkSmem {
    Buf<CC<DK>> b;
    // the column-contracted sums in [channel x token] accumulator tiles
    // (lane (token n, g4) of tile t: channels 16 t + 4 g4 + e):
    // [0] Sd dO^T, [1] Sd dX^T, [2] L U^T
    alignas(16) f32x4 RED[3][DK / 16][WAVE];
    alignas(16) f32x4 RT[2][WAVE];       // dU X^T, dO U^T (lane (i, g4): rows 4 g4 + e)
    alignas(16) float DT[16][17], DP[16][17], DM[16][17], W[16][17], DA[16][17];
    alignas(16) float RG[4][DK];         // per wave: sum over its columns of L o Sd
    alignas(16) float GQ[DK];            // sum over the tokens of QE o (dO Sd^T) - KE o (dX Sd^T)
    alignas(16) float DB[16];
};

}  // namespace bwdm

// One workgroup (four waves) per (chunk slot, head); sized for two
// workgroups per compute unit.
template <int DK, int DV>
__global__ __launch_bounds__(256, 2)
void kda_bwd_chunk(const bwdm::ChunkParams p)
{
    using namespace bwdm;
    using C = CC<DK>;
    constexpr int NT16 = DK / 16, NS = DK / 32;
    __shared__ ChunkSmem<DK, DV> sm;
    Buf<C> &B = sm.b;
    // the log-decay terms dx [token][channel] reuse the -KE and QE hi rows,
    // which nothing reads after the column blocks
    static_assert(sizeof(float) * 16 * (DK + 4) <= sizeof(B.NK) + sizeof(B.QH), "dx scratch");
    static_assert(offsetof(Buf<C>, QH) == offsetof(Buf<C>, NK) + sizeof(B.NK), "dx scratch");
    float (*DXS)[DK + 4] = reinterpret_cast<float (*)[DK + 4]>(&B.NK[0][0]);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, g4 = lane >> 4;
    const int H = p.H;
    const int64_t slot = blockIdx.x / H;
    const int h = blockIdx.x % H;
    // the slot's sequence: chunk c of sequence n has slot bos_n / 16 + n + c
    auto bos_of = [&](int s) -> int64_t {
        if (!p.cu_seqlens) return (int64_t)s * p.seqlen;
        const int32_t c0 = p.cu_seqlens[s];
        return c0 < 0 ? 0 : (c0 > p.n_tokens ? p.n_tokens : c0);
    };
    int lo = 0, hi = p.n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (bos_of(mid) / 16 + mid <= slot) lo = mid;
        else hi = mid - 1;
    }
    const int n = lo;
    const int64_t bos = bos_of(n);
    int64_t T;
    if (p.cu_seqlens) {
        const int32_t c1 = p.cu_seqlens[n + 1];
        const int64_t a1 = c1 < 0 ? 0 : (c1 > p.n_tokens ? p.n_tokens : c1);
        T = a1 > bos ? a1 - bos : 0;
    } else {
        T = p.seqlen;
    }
    const int64_t c = slot - (bos / 16 + n);
    if (c < 0 || c * 16 >= T) return;
    const int64_t tok0 = uniform64(bos + c * 16);
    const int nt = __builtin_amdgcn_readfirstlane((int)(T - c * 16 < 16 ? T - c * 16 : 16));
    // q, k, v, dO of the chunk, rows past its end read as zero
    const int krow = H * DK * 2, vrow = H * DV * 2;      // bytes per token (< 2^27, host)
    const rsrc_t rq = make_rsrc(p.q + tok0 * H * DK, nt * krow);
    const rsrc_t rk = make_rsrc(p.k + tok0 * H * DK, nt * krow);
    const rsrc_t rv = make_rsrc(p.v + tok0 * H * DV, nt * vrow);
    const rsrc_t ro = make_rsrc(p.dO + tok0 * H * DV, nt * vrow);

    // The column blocks (step 3) take the chunk-start state, as the decayed
    // Sd hi / lo operands the checkpointing forward split and stored, and the
    // exit cotangent L one block of 16 columns at a time, wave w taking
    // blocks w, w + 4, ...  The first block's checkpoint tiles and v, dO
    // values are requested before the operand build, so that their latency
    // overlaps it; a later block's Sd (L) tiles as soon as the previous
    // block's have been taken up (L: split), into the same registers.
    constexpr int NCB = DV / 16, NIT = (NCB + 3) / 4;
    typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
    const f32x4 *cs = reinterpret_cast<const f32x4 *>(p.Sck + (slot * H + h) * (int64_t)(DK * DV));
    const f32x4 *cl = reinterpret_cast<const f32x4 *>(p.Lck + (slot * H + h) * (int64_t)(DK * DV));
    bf16x8 shn[NS], sln[NS];              // Sd hi / lo operands, as the forward wrote them
    f32x4 Ln[NT16];
    u16x4 vbn, obn;                       // v, dO of column 16 cb + j, tokens 4 g4 + i
    u32x2 o4n;                            // dO of token j, columns 16 cb + 4 g4 .. + 3
    // checkpoints: read once, streamed
    auto fetch_l = [&](int cb) {
#pragma unroll
        for (int t = 0; t < NT16; ++t) Ln[t] = __builtin_nontemporal_load(&cl[(cb * NT16 + t) * WAVE + lane]);
    };
    // (v and dO first: their 16-bit halves are packed as soon as they arrive)
    auto fetch_s = [&](int cb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int off = (4 * g4 + i) * vrow + (h * DV + 16 * cb + j) * 2;
            vbn[i] = __builtin_amdgcn_raw_buffer_load_b16(rv, off, 0, 0);
            obn[i] = __builtin_amdgcn_raw_buffer_load_b16(ro, off, 0, 0);
        }
        o4n = bload64(ro, j * vrow + (h * DV + 16 * cb + 4 * g4) * 2);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            shn[s] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(&cs[(cb * NT16 + 2 * s) * WAVE + lane])));
            sln[s] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(&cs[(cb * NT16 + 2 * s + 1) * WAVE + lane])));
        }
    };
    // 1. chunk operands (builder waves); sums cleared.  The builders' raw
    // inputs are requested before the checkpoint tiles: loads complete in
    // order, so the build then waits only for its own inputs.
    Raw<C> r;
    if (wave < C::NBW)
        load_raw<C>(r, p.q, p.k, p.v, p.g, p.beta, tok0, nt, 0, H, h, DV, 0, wave, lane, tid);
    if (NCB >= 4 || wave < NCB) {
        fetch_s(wave);
        fetch_l(wave);
    }
    if (wave < C::NBW) build<C>(B, r, wave, lane, tid, 1.f);
    for (int e = tid; e < 3 * NT16 * WAVE; e += 256) (&sm.RED[0][0][0])[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int e = tid; e < 2 * WAVE; e += 256) (&sm.RT[0][0])[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    // 2. helpers: T^T, P^T, (I + A)^{-1} and KE Kd^T
    if (wave == 0) helper<C, 0>(B, lane);
    else if (wave == 1) helper<C, 1>(B, lane);
    __syncthreads();

    // 3. blocks of 16 value columns, wave w taking blocks w, w + 4, ...  The
    // sums are split in four groups of channel tiles; in round r wave w adds
    // the products of all its blocks into group (w + r) % 4 (and the wave of
    // group 0 also adds dU X^T, dO U^T), so no two waves touch the same sums
    // between barriers.  The row sums of L o Sd over the columns are the
    // diagonal of L Sd^T, formed per channel tile from the same transposed
    // tiles as the other sums and kept per lane until the column phase ends.
    {
        constexpr int TPQ = NT16 >= 4 ? NT16 / 4 : 1;   // channel tiles per group
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const NegEye ne = neg_eye(lane);
        const bf16x8 eyeA = eye_half(lane, 0), eyeB = eye_half(lane, 1);
        // lane (n, g4) keeps the diagonal entry of row n: element n % 4 of g4 = n / 4
        const int e3 = j & 3;
        const float m0 = e3 == 0 ? 1.f : 0.f, m1 = e3 == 1 ? 1.f : 0.f;
        const float m2 = e3 == 2 ? 1.f : 0.f, m3 = e3 == 3 ? 1.f : 0.f;
        // T rows [Th | Th], [Tl | Tl] read out of the T^T rows
        bf16x4 th4, tl4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            th4[e] = B.TH[4 * g4 + e][8 * (j >> 2) + (j & 3)];
            tl4[e] = B.TL[4 * g4 + e][8 * (j >> 2) + (j & 3)];
        }
        const bf16x8 t2h = cat(th4, th4), t2l = cat(tl4, tl4);
        const bf16x8 tth = ld8b(&B.TH[j][8 * g4]), ttl = ld8b(&B.TL[j][8 * g4]);
        const bf16x8 pth = ld8b(&B.PH[j][8 * g4]);
        float DG[NT16];
#pragma unroll
        for (int t = 0; t < NT16; ++t) DG[t] = 0.f;
        // Every block of the wave first (the first block's tiles were fetched
        // before the operand build, a later block's at its start), then four
        // rounds over the channel groups, each taking the products of all the
        // wave's blocks.  (Unrolled: the prefetched tiles are then not held
        // across a back edge.)
        bf16x8 sh[NIT][NS], sl[NIT][NS], lh[NIT][NS], ll[NIT][NS];
        bf16x8 doo[NIT], buh[NIT], bul[NIT], bxh[NIT], bxl[NIT];
        f32x4 dT = zero, dP = zero;                       // over the wave's blocks
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int cb = wave + 4 * it;
            if (cb >= NCB) break;                         // uniform over the wave
            // the next block's S and L tiles are requested as soon as this
            // block's have been split (into the same registers)
            const bool more = it + 1 < NIT && cb + 4 < NCB;
            const bf16x4 v4 = __builtin_bit_cast(bf16x4, vbn), d4 = __builtin_bit_cast(bf16x4, obn);
            const bf16x4 o4 = __builtin_bit_cast(bf16x4, o4n);
            doo[it] = cat(o4, o4);
            // Sd hi / lo, as the checkpointing forward split it
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                sh[it][s] = shn[s];
                sl[it][s] = sln[s];
            }
            if (more) fetch_s(cb + 4);
            // X = V - KE Sd
            f32x4 x = {(float)v4[0], (float)v4[1], (float)v4[2], (float)v4[3]};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const bf16x8 nk = ld8b(&B.NK[j][32 * s + 8 * g4]);
                x = mma32(nk, sh[it][s], x);
                x = mma32(nk, sl[it][s], x);
            }
            bf16x4 xh, xl;
            split4(x, ne, xh, xl);
            const bf16x8 xhl = cat(xh, xl);
            // U = T X
            f32x4 u = mma32(t2h, xhl, zero);
            u = mma32(t2l, xhl, u);
#pragma unroll
            for (int s = 0; s < NS; ++s) split8(Ln[2 * s], Ln[2 * s + 1], ne, lh[it][s], ll[it][s]);
            if (more) fetch_l(cb + 4);
            // dU = P^T dO + Kd L
            f32x4 du = mma32(pth, cat(d4, d4), zero);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const int kk = 32 * s + 8 * g4;
                const bf16x8 dh = ld8b(&B.DH[j][kk]), dl = ld8b(&B.DL[j][kk]);
                du = mma32(dh, lh[it][s], du);
                du = mma32(dl, lh[it][s], du);
                du = mma32(dh, ll[it][s], du);
            }
            bf16x4 uh, ul, duh, dul;
            split4(u, ne, uh, ul);
            split4(du, ne, duh, dul);
            const bf16x8 uhl = cat(uh, ul), duhl = cat(duh, dul);
            // dX = T^T dU
            f32x4 dx = mma32(tth, duhl, zero);
            dx = mma32(ttl, duhl, dx);
            bf16x4 dxh, dxl;
            split4(dx, ne, dxh, dxl);
            // transposed tiles (value columns as rows): lane (token n, g4)
            // holds columns 16 cb + 4 g4 .. + 3 of token n
            bf16x4 xth, xtl, uth, utl, duth, dutl, dxth, dxtl;
            const bf16x8 dxhl = cat(dxh, dxl);
            xth = to_bf16x4(mma32(xhl, eyeA, zero));
            xtl = to_bf16x4(mma32(xhl, eyeB, zero));
            uth = to_bf16x4(mma32(uhl, eyeA, zero));
            utl = to_bf16x4(mma32(uhl, eyeB, zero));
            duth = to_bf16x4(mma32(duhl, eyeA, zero));
            dutl = to_bf16x4(mma32(duhl, eyeB, zero));
            dxth = to_bf16x4(mma32(dxhl, eyeA, zero));
            dxtl = to_bf16x4(mma32(dxhl, eyeB, zero));
            // dU X^T and dO U^T (16 x 16, lane (i, g4): rows 4 g4 + e)
            dT = mma32(cat(duth, dutl), cat(xth, xth), dT);
            dT = mma32(cat(duth, dutl), cat(xtl, xtl), dT);
            dP = mma32(doo[it], cat(uth, utl), dP);
            buh[it] = cat(uth, uth); bul[it] = cat(utl, utl);
            bxh[it] = cat(dxth, dxth); bxl[it] = cat(dxtl, dxtl);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int grp = (wave + r) & 3;
#pragma unroll
            for (int G = 0; G < 4; ++G) {
                if (G != grp || G * TPQ >= NT16 || wave >= NCB) continue;
#pragma unroll
                for (int tt = 0; tt < TPQ; ++tt) {
                    const int t = G * TPQ + tt, s = t >> 1;
                    f32x4 y1 = sm.RED[0][t][lane], y2 = sm.RED[1][t][lane];
                    f32x4 kd = sm.RED[2][t][lane];
                    f32x4 dd = zero;
                    // tile t is half t % 2 of the [tile 2s | tile 2s + 1] operands
                    const bf16x8 ey = (t & 1) ? eyeB : eyeA;
#pragma unroll
                    for (int it = 0; it < NIT; ++it) {
                        if (wave + 4 * it >= NCB) break;   // uniform over the wave
                        // Sd and L tile t transposed, hi and lo parts
                        const bf16x4 sth = to_bf16x4(mma32(sh[it][s], ey, zero));
                        const bf16x4 stl = to_bf16x4(mma32(sl[it][s], ey, zero));
                        const bf16x4 lth = to_bf16x4(mma32(lh[it][s], ey, zero));
                        const bf16x4 ltl = to_bf16x4(mma32(ll[it][s], ey, zero));
                        const bf16x8 sa = cat(sth, stl), la = cat(lth, ltl);
                        // diag(L Sd^T): lane (n, g4) holds entries (4 g4 + e, n)
                        dd = mma32(la, cat(sth, sth), dd);
                        dd = mma32(la, cat(stl, stl), dd);
                        y1 = mma32(sa, doo[it], y1);                   // Sd dO^T
                        y2 = mma32(sa, bxh[it], y2);                   // Sd dX^T
                        y2 = mma32(sa, bxl[it], y2);
                        kd = mma32(la, buh[it], kd);                   // L U^T
                        kd = mma32(la, bul[it], kd);
                    }
                    sm.RED[0][t][lane] = y1;
                    sm.RED[1][t][lane] = y2;
                    sm.RED[2][t][lane] = kd;
                    DG[t] += (dd[0] * m0 + dd[1] * m1) + (dd[2] * m2 + dd[3] * m3);
                }
            }
            if (grp == 0 && wave < NCB) {
                sm.RT[0][lane] += dT;
                sm.RT[1][lane] += dP;
            }
            __syncthreads();
        }
        if ((j >> 2) == g4) {
#pragma unroll
            for (int t = 0; t < NT16; ++t) sm.RG[wave][16 * t + j] = DG[t];
        }
    }
    // the q, k values of step 5 (wave w takes channel tiles w, w + 4, ...),
    // requested here so that they arrive during step 4
    constexpr int NTW = (NT16 + 3) / 4;
    uint16_t pq[NTW][4], pk[NTW][4];
    u32x2 pq4[NTW], pk4[NTW];
#pragma unroll
    for (int w2 = 0; w2 < NTW; ++w2) {
        const int t = wave + 4 * w2;
        if (t >= NT16) break;              // uniform over the wave
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int off = (4 * st + g4) * krow + (h * DK + 16 * t + j) * 2;
            pq[w2][st] = __builtin_amdgcn_raw_buffer_load_b16(rq, off, 0, 0);
            pk[w2][st] = __builtin_amdgcn_raw_buffer_load_b16(rk, off, 0, 0);
        }
        const int off = j * krow + (h * DK + 16 * t + 4 * g4) * 2;
        pq4[w2] = bload64(rq, off);
        pk4[w2] = bload64(rk, off);
    }
    // 4. through T = M Diag(beta) and A = strict_lower(Diag(beta) KE Kd^T)
    const int r16 = tid >> 4, i16 = tid & 15;
    if (tid < 64) {
        const f32x4 a = sm.RT[0][tid], b = sm.RT[1][tid];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sm.DT[4 * g4 + e][j] = a[e];
            sm.DP[4 * g4 + e][j] = b[e];
        }
    }
    __syncthreads();
    {
        float w = 0.f;                                                // W = M^T dM,
#pragma unroll
        for (int q = 0; q < 16; ++q) w = __builtin_fmaf(B.MI[q][r16], sm.DT[q][i16], w);
        sm.W[r16][i16] = w * B.BETA[i16];                             // dM = dT Diag(beta)
    }
    __syncthreads();
    {
        float a = 0.f;                                                // dA = -W M^T
#pragma unroll
        for (int q = 0; q < 16; ++q) a = __builtin_fmaf(sm.W[r16][q], B.MI[i16][q], a);
        const float da = i16 < r16 ? -a : 0.f;
        sm.DM[r16][i16] = da;                                         // dA itself, for dbeta
        sm.DA[r16][i16] = da * B.BETA[r16];                           // Diag(beta) dA
        if (i16 > r16) sm.DP[r16][i16] = 0.f;                         // P lower incl.
    }
    __syncthreads();
    // dbeta (read after the barrier that ends step 5)
    if (tid < 16) {
        float b = 0.f;
        for (int q = 0; q < 16; ++q) b = __builtin_fmaf(sm.DT[q][tid], B.MI[q][tid], b);
        for (int q = 0; q < 16; ++q) b = __builtin_fmaf(sm.DM[tid][q], B.KK[tid][q], b);
        sm.DB[tid] = b;
    }
    // 5. dQE, dKE, dKd as [channel x token] tiles (fp32 matrix cores), then
    // dq, dk and the log-decay terms; QE, KE, Kd are re-formed from q, k and
    // the exponents
#pragma unroll
    for (int w2 = 0; w2 < NTW; ++w2) {
        const int t = wave + 4 * w2;
        if (t >= NT16) break;              // uniform over the wave
        f32x4 q1 = {0.f, 0.f, 0.f, 0.f}, q2 = q1, q3 = q1;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int kk = 4 * st + g4;                               // token index i
            const int ch = 16 * t + j;
            const float qv = u16_to_f(pq[w2][st]);
            const float kv = u16_to_f(pk[w2][st]);
            const float x = B.GX[kk][ch];
            const float E = fast_exp2(x), F = fast_exp2(-x);
            q1 = mma4(kv * F, sm.DP[j][kk], q1);                      // Kd^T dP^T
            q2 = mma4(kv * F, sm.DA[j][kk], q2);                      // Kd^T dA^T
            q3 = mma4(qv * E, sm.DP[kk][j], q3);                      // QE^T dP
            q3 = mma4(kv * E, sm.DA[kk][j], q3);                      // + KE^T dA
        }
        const bf16x4 q4 = __builtin_bit_cast(bf16x4, pq4[w2]);
        const bf16x4 k4 = __builtin_bit_cast(bf16x4, pk4[w2]);
        // (read into registers first: the log-decay terms are written over
        // LDS rows the compiler cannot tell apart from the sums)
        const f32x4 Y1 = sm.RED[0][t][lane], Y2 = sm.RED[1][t][lane], KD = sm.RED[2][t][lane];
        const f32x4 GXv = *reinterpret_cast<const f32x4 *>(&B.GX[j][16 * t + 4 * g4]);   // log2 units, >= 0
        f32x4 dqv, dkv, gqv, dxv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float y1 = Y1[e], y2 = Y2[e];
            const float dqe = y1 + q1[e];
            const float dke = -y2 + q2[e];
            const float dkd = KD[e] + q3[e];
            const float E = fast_exp2(GXv[e]), F = fast_exp2(-GXv[e]);
            const float qe = (float)q4[e] * E, ke = (float)k4[e] * E, kd = (float)k4[e] * F;
            dqv[e] = dqe * E;
            dkv[e] = dke * E + dkd * F;
            gqv[e] = qe * y1 - ke * y2;
            dxv[e] = dqe * qe + dke * ke - dkd * kd;
        }
        *reinterpret_cast<f32x4 *>(&DXS[j][16 * t + 4 * g4]) = dxv;
        if (j < nt) {
            const int64_t o = ((tok0 + j) * H + h) * DK + 16 * t + 4 * g4;
            *reinterpret_cast<f32x4 *>(p.dq + o) = dqv;
            *reinterpret_cast<f32x4 *>(p.dk + o) = dkv;
        }
        // sums over the 16 tokens (the lanes of a row)
#pragma unroll
        for (int e = 0; e < 4; ++e) gqv[e] = group_sum<16>(gqv[e]);
        if (j == 0) *reinterpret_cast<f32x4 *>(&sm.GQ[16 * t + 4 * g4]) = gqv;
    }
    __syncthreads();
    // 6. dg: x_r = Gc_r - Gc_16 gives dGc_r = dx_r (r < 15) and the chunk
    // total dGc_16 = gamma dgamma - sum_{r < 15} dx_r; dg_s = sum_{r >= s} dGc_r,
    // with gamma dgamma = sum_j dSd o Sd = L o Sd + QE o (dO Sd^T) - KE o (dX Sd^T)
    // (every thread: 256 / d_k threads per channel, each storing 16 d_k / 256
    // of the tokens)
    {
        constexpr int NPC = 256 / DK, TPT = 16 / NPC;
        static_assert(NPC * DK == 256 && NPC * TPT == 16, "dg mapping");
        const int ch = tid % DK, r0 = (tid / DK) * TPT;
        float dx[16], tot = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dx[r] = DXS[r][ch];
            tot += dx[r];
        }
        float acc = (sm.RG[0][ch] + sm.RG[1][ch]) + (sm.RG[2][ch] + sm.RG[3][ch]) + sm.GQ[ch] - tot + dx[15];
        float *dgp = p.dg + ((tok0 + r0) * H + h) * DK + ch;
        const int64_t step = (int64_t)H * DK;
#pragma unroll
        for (int r = 15; r >= 0; --r) {
            if (r < 15) acc += dx[r];
            if (r >= r0 && r < r0 + TPT && r < nt) dgp[(r - r0) * step] = acc;
        }
    }
    if (tid < nt) p.db[(tok0 + tid) * H + h] = sm.DB[tid];
}

template <int DK, int DV>
static hipError_t launch_bwd_mfma_t(const BwdArgs &a)
{
    using namespace bwdm;
    constexpr int NW = DV / 16 < 4 ? (DV / 16 < DK / 16 ? DV / 16 : DK / 16)
                                   : (4 < DK / 16 ? 4 : DK / 16);
    using SCf = SC<DK, NW>;
    constexpr int NB = DV / SCf::BV;
    static_assert(sizeof(Smem<SCf>) <= 160 * 1024, "sweep LDS");
    static_assert(sizeof(ChunkSmem<DK, DV>) <= 160 * 1024, "chunk LDS");
    const int64_t chains = (int64_t)a.n_seqs * a.H;
    if (chains == 0) return hipSuccess;
    hipStream_t st = (hipStream_t)a.stream;
    SweepParams sp{};
    sp.q = (const bf16 *)a.q; sp.k = (const bf16 *)a.k; sp.dO = (const bf16 *)a.dO;
    sp.g = a.g; sp.beta = a.beta; sp.dST = a.dST; sp.cu_seqlens = a.cu_seqlens;
    sp.seqlen = a.seqlen; sp.n_tokens = (int32_t)a.n_tokens;
    sp.n_chains = (int32_t)chains; sp.chains8 = (int32_t)(((chains + 7) / 8) * 8); sp.H = a.H;
    sp.Lck = a.part; sp.dv = a.dv; sp.dS0 = a.dS0;
    const int64_t grid = (int64_t)sp.chains8 * NB;
    hipLaunchKernelGGL((kda_bwd_sweep_mfma<DK, DV, NW>), dim3((unsigned)grid), dim3(SCf::NT), 0,
                       st, sp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t g2 = a.n_slots * a.H;
    if (g2 == 0) return hipSuccess;
    ChunkParams cp{};
    cp.q = (const bf16 *)a.q; cp.k = (const bf16 *)a.k; cp.v = (const bf16 *)a.v;
    cp.dO = (const bf16 *)a.dO; cp.g = a.g; cp.beta = a.beta; cp.cu_seqlens = a.cu_seqlens;
    cp.n_seqs = a.n_seqs; cp.seqlen = a.seqlen; cp.n_tokens = (int32_t)a.n_tokens; cp.H = a.H;
    cp.Sck = a.ckpt; cp.Lck = a.part;
    cp.dq = a.dq; cp.dk = a.dk; cp.dg = a.dg; cp.db = a.dbeta;
    hipLaunchKernelGGL((kda_bwd_chunk<DK, DV>), dim3((unsigned)g2), dim3(256), 0, st, cp);
    return hipGetLastError();
}

template <typename TI, int DK, int DV>
static hipError_t launch_bwd_t(const BwdArgs &a)
{
    constexpr int BV = DV >= 64 ? 64 : DV;
    constexpr int NB = DV / BV;
    static_assert(sizeof(bwd::SweepSmem<DK, BV>) <= 160 * 1024, "LDS");
    static_assert(sizeof(bwd::FinishSmem<DK>) <= 160 * 1024, "LDS");
    const int64_t chains = (int64_t)a.n_seqs * a.H;
    if (chains == 0) return hipSuccess;
    hipStream_t st = (hipStream_t)a.stream;
    hipLaunchKernelGGL((kda_bwd_sweep<TI, DK, DV, BV>), dim3((unsigned)(chains * NB)),
                       dim3(bwd::NT), 0, st, (const TI *)a.q, (const TI *)a.k, (const TI *)a.v,
                       a.g, a.beta, (const TI *)a.dO, a.dST, a.cu_seqlens, a.seqlen,
                       (int32_t)a.n_tokens, a.H, a.ckpt, a.part, a.dv, a.dS0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t grid = a.n_slots * a.H;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((kda_bwd_finish<TI, DK, NB>), dim3((unsigned)grid), dim3(bwd::NT), 0, st,
                       (const TI *)a.q, (const TI *)a.k, a.g, a.beta, a.cu_seqlens, a.n_seqs,
                       a.seqlen, (int32_t)a.n_tokens, a.H, a.part, a.dq, a.dk, a.dg, a.dbeta);
    return hipGetLastError();
}

size_t bwd_part_floats(int32_t d_k, int32_t d_v)
{
    // vector-ALU path: per-block partial sums; matrix-core path: the exit
    // cotangent of the chunk (d_k x d_v)
    const int BV = d_v >= 64 ? 64 : d_v;
    const int NB = d_v / BV;
    const size_t part = (size_t)NB * (3 * bwd::C * d_k + 2 * bwd::C * bwd::C + d_k);
    const size_t lck = (size_t)d_k * d_v;
    return part > lck ? part : lck;
}

template <typename TI>
static hipError_t dispatch_bwd(const BwdArgs &a)
{
#define KDA_BWD_CASE(DK_, DV_) \
    if (a.d_k == DK_ && a.d_v == DV_) return launch_bwd_t<TI, DK_, DV_>(a);
    KDA_BWD_CASE(16, 16) KDA_BWD_CASE(16, 32) KDA_BWD_CASE(16, 64) KDA_BWD_CASE(16, 128)
    KDA_BWD_CASE(32, 16) KDA_BWD_CASE(32, 32) KDA_BWD_CASE(32, 64) KDA_BWD_CASE(32, 128)
    KDA_BWD_CASE(64, 16) KDA_BWD_CASE(64, 32) KDA_BWD_CASE(64, 64) KDA_BWD_CASE(64, 128)
    KDA_BWD_CASE(128, 16) KDA_BWD_CASE(128, 32) KDA_BWD_CASE(128, 64) KDA_BWD_CASE(128, 128)
#undef KDA_BWD_CASE
    return hipErrorInvalidValue;
}

static hipError_t dispatch_bwd_mfma(const BwdArgs &a)
{
#define KDA_BWD_CASE(DK_, DV_) \
    if (a.d_k == DK_ && a.d_v == DV_) return launch_bwd_mfma_t<DK_, DV_>(a);
    KDA_BWD_CASE(32, 16) KDA_BWD_CASE(32, 32) KDA_BWD_CASE(32, 64) KDA_BWD_CASE(32, 128)
    KDA_BWD_CASE(64, 16) KDA_BWD_CASE(64, 32) KDA_BWD_CASE(64, 64) KDA_BWD_CASE(64, 128)
    KDA_BWD_CASE(128, 16) KDA_BWD_CASE(128, 32) KDA_BWD_CASE(128, 64) KDA_BWD_CASE(128, 128)
#undef KDA_BWD_CASE
    return hipErrorInvalidValue;
}

// bf16 inputs with d_k >= 32 take the matrix-core kernels; fp32 inputs (the
// precision reference) and d_k = 16 the vector-ALU ones
hipError_t launch_bwd(const BwdArgs &a)
{
    if (a.in_bf16 && a.d_k >= 32) return dispatch_bwd_mfma(a);
    return a.in_bf16 ? dispatch_bwd<bf16>(a) : dispatch_bwd<float>(a);
}

}  // namespace kda
