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
// state does: kda_bwd_sweep runs one workgroup per (sequence, head, block of
// columns) backwards over the chunks, from the chunk-start states that the
// prefill kernel checkpointed, and writes its dv and dS0 columns directly.
// The products that contract over d_v (dO Sd^T, dX Sd^T, U L^T, dU X^T,
// dO U^T, dgamma) only feed the per-chunk gradients; every block writes its
// partial sums, and kda_bwd_finish, one workgroup per (chunk, head), adds
// them up and forms dq, dk, dg and dbeta, all chunks in parallel.
//
// Arithmetic is fp32 on the vector ALU throughout (no matrix cores, no
// bf16 operands); products are LDS-staged, each thread accumulating a small
// tile of outputs.
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
    const int BV = d_v >= 64 ? 64 : d_v;
    const int NB = d_v / BV;
    return (size_t)NB * (3 * bwd::C * d_k + 2 * bwd::C * bwd::C + d_k);
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

hipError_t launch_bwd(const BwdArgs &a)
{
    return a.in_bf16 ? dispatch_bwd<bf16>(a) : dispatch_bwd<float>(a);
}

}  // namespace kda
