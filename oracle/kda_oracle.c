/*
 * KDA oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64, token-by-token evaluation of the Kimi Delta Attention
 * recurrence.  Only the test-suite, the smoke check and the bench's CPU
 * baseline may load this library; the product path never does.
 *
 * Definition followed (Kimi K3 architecture walkthrough, mhpq.cn/news/56770,
 * section "KDA 到底在算什么", the state-update equation and the figure
 * caption that orders its steps): per head, with a d_k x d_v state S whose
 * rows are key channels,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t ,                alpha_t = exp(g_t) per key channel
 *
 * (the alpha = exp(g) parameterisation is the one in the K3-on-TPU essay,
 * blog.higcp.com, section "KDA + Gated MLA", lower-bounded decay).
 * The code evaluates the same map in its rank-1 form: decay the rows, form
 * u = beta (v - S'^T k) against the decayed state S', add k u^T, then read
 * o = S^T q.  Expanding (I - b k k^T) S' + b k v^T = S' + b k (v - S'^T k)^T
 * shows the two are the same expression.
 *
 * No blocking, no reordering: one token at a time, one (sequence, head) per
 * OpenMP iteration.  kda_oracle_vjp (at the end) gives the reverse-mode
 * gradients of the same map, token by token in reverse.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One (sequence, head) chain.
 * q, k, g : element (t, c) at base[t * ld_k + c]      (t < T, c < dk)
 * v       : element (t, j) at base[t * ld_v + j]      (j < dv)
 * beta    : element t      at base[t * ld_b]
 * S       : [dk][dv] row-major fp64, in: entry state, out: final state
 * o       : element (t, j) at base[t * ld_o + j], fp64 (may be NULL)      */
static void chain(int64_t T, int dk, int dv,
                  const float *q, const float *k, const float *v,
                  const float *g, const float *beta,
                  int64_t ld_k, int64_t ld_v, int64_t ld_b,
                  double *S, double *o, int64_t ld_o,
                  double *w /* scratch [dv] */)
{
    for (int64_t t = 0; t < T; ++t) {
        const float *qt = q + t * ld_k, *kt = k + t * ld_k, *gt = g + t * ld_k;
        const float *vt = v + t * ld_v;
        const double b = (double)beta[t * ld_b];
        /* S' = Diag(exp(g_t)) S : row i scaled by its channel's retention */
        for (int i = 0; i < dk; ++i) {
            const double a = exp((double)gt[i]);
            double *row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) row[j] *= a;
        }
        /* w = S'^T k */
        for (int j = 0; j < dv; ++j) w[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double ki = (double)kt[i];
            const double *row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) w[j] += row[j] * ki;
        }
        /* u = beta (v - w), stored in w */
        for (int j = 0; j < dv; ++j) w[j] = b * ((double)vt[j] - w[j]);
        /* S = S' + k u^T */
        for (int i = 0; i < dk; ++i) {
            const double ki = (double)kt[i];
            double *row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) row[j] += ki * w[j];
        }
        /* o_t = S^T q */
        if (o) {
            double *ot = o + t * ld_o;
            for (int j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int i = 0; i < dk; ++i) {
                const double qi = (double)qt[i];
                const double *row = S + (size_t)i * dv;
                for (int j = 0; j < dv; ++j) ot[j] += row[j] * qi;
            }
        }
    }
}

/* Packed varlen batch.
 * q, k, g : [N, H, dk] fp32; v : [N, H, dv] fp32; beta : [N, H] fp32
 * S0      : [n_seqs, H, dk, dv] fp32 or NULL (zeros)
 * cu      : int32 [n_seqs + 1], non-decreasing, cu[0] = 0
 * o       : [N, H, dv] fp64 out (may be NULL); S_T : [n_seqs, H, dk, dv] fp64 out
 * Returns the number of threads used.                                      */
int kda_oracle_fwd(const float *q, const float *k, const float *v,
                   const float *g, const float *beta, const float *S0,
                   const int32_t *cu, int n_seqs, int H, int dk, int dv,
                   double *o, double *S_T, int n_threads)
{
    int used = 1;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
    const int64_t pairs = (int64_t)n_seqs * H;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double *w = (double *)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < pairs; ++p) {
            const int n = (int)(p / H), h = (int)(p % H);
            const int64_t t0 = cu[n], T = (int64_t)cu[n + 1] - cu[n];
            double *S = S_T + ((size_t)n * H + h) * (size_t)dk * dv;
            if (S0) {
                const float *s0 = S0 + ((size_t)n * H + h) * (size_t)dk * dv;
                for (size_t e = 0; e < (size_t)dk * dv; ++e) S[e] = (double)s0[e];
            } else {
                memset(S, 0, sizeof(double) * (size_t)dk * dv);
            }
            chain(T, dk, dv,
                  q + (t0 * H + h) * dk, k + (t0 * H + h) * dk,
                  v + (t0 * H + h) * dv, g + (t0 * H + h) * dk,
                  beta + t0 * H + h,
                  (int64_t)H * dk, (int64_t)H * dv, H,
                  S, o ? o + (t0 * H + h) * dv : NULL, (int64_t)H * dv, w);
        }
        free(w);
    }
    return used;
}

/* One chain with contiguous per-head arrays: q, k, g [T, dk]; v [T, dv];
 * beta [T]; S (in/out) [dk, dv] fp64; o [T, dv] fp64 or NULL.  Used for
 * sampled checks on single heads of large batches.                         */
void kda_oracle_head(int64_t T, int dk, int dv,
                     const float *q, const float *k, const float *v,
                     const float *g, const float *beta, double *S, double *o)
{
    double *w = (double *)malloc(sizeof(double) * (size_t)dv);
    chain(T, dk, dv, q, k, v, g, beta, dk, dv, 1, S, o, dv, w);
    free(w);
}

/* Reverse-mode gradients of one chain (the same recurrence), fp64.
 * Given cotangents dO of every o_t and dST of the final state, walk the
 * tokens backwards applying the chain rule to the five lines of the rank-1
 * form  S'_t = Diag(exp(g_t)) S_{t-1};  w_t = S'_t^T k_t;
 * u_t = beta_t (v_t - w_t);  S_t = S'_t + k_t u_t^T;  o_t = S_t^T q_t
 * in reverse order, with dS the cotangent of S_t:
 *     dS += q_t dO_t^T;       dq_t = S_t dO_t
 *     du  = dS^T k_t;         dk_t = dS u_t;     dv_t = beta_t du
 *     dbeta_t = (v_t - w_t) . du;                dw = -beta_t du
 *     dS' = dS + k_t dw^T;    dk_t += S'_t dw;   dg_t = rowsum(dS' o S'_t)
 *     dS  = Diag(exp(g_t)) dS'
 * and dS0 = dS at the end.  (A custom-VJP backward is part of the KDA kernel
 * suite in the K3-on-TPU essay, blog.higcp.com, the section on the existing
 * TPU kernel.)  Every state S_0 .. S_T is kept (Sall, [T + 1][dk][dv]); S'_t
 * is re-formed from S_{t-1} with the forward's own operations.
 * Layouts as in chain(); dO like v; gradients fp64 with the inputs' layouts
 * (dq, dk, dg like q; dv like v; dbeta like beta).                          */
static void vjp_chain(int64_t T, int dk, int dv,
                      const float *q, const float *k, const float *v,
                      const float *g, const float *beta, const float *dO,
                      int64_t ld_k, int64_t ld_v, int64_t ld_b,
                      const float *S0, const float *dST,
                      double *dq, double *dkk, double *dvv, double *dg, double *db,
                      double *dS0,
                      double *Sall, double *W, double *U, double *Sp, double *dS,
                      double *du)
{
    const size_t ss = (size_t)dk * dv;
    /* forward, keeping S_t and w_t, u_t */
    for (size_t e = 0; e < ss; ++e) Sall[e] = S0 ? (double)S0[e] : 0.0;
    for (int64_t t = 0; t < T; ++t) {
        const float *kt = k + t * ld_k, *gt = g + t * ld_k, *vt = v + t * ld_v;
        const double b = (double)beta[t * ld_b];
        const double *Sprev = Sall + (size_t)t * ss;
        double *S = Sall + (size_t)(t + 1) * ss;
        double *w = W + (size_t)t * dv, *u = U + (size_t)t * dv;
        for (int i = 0; i < dk; ++i) {
            const double a = exp((double)gt[i]);
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] = Sprev[(size_t)i * dv + j] * a;
        }
        for (int j = 0; j < dv; ++j) w[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) w[j] += S[(size_t)i * dv + j] * (double)kt[i];
        for (int j = 0; j < dv; ++j) u[j] = b * ((double)vt[j] - w[j]);
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += (double)kt[i] * u[j];
    }
    /* backward */
    for (size_t e = 0; e < ss; ++e) dS[e] = dST ? (double)dST[e] : 0.0;
    for (int64_t t = T - 1; t >= 0; --t) {
        const float *qt = q + t * ld_k, *kt = k + t * ld_k, *gt = g + t * ld_k;
        const float *vt = v + t * ld_v, *dot = dO + t * ld_v;
        const double b = (double)beta[t * ld_b];
        const double *S = Sall + (size_t)(t + 1) * ss, *Sprev = Sall + (size_t)t * ss;
        const double *w = W + (size_t)t * dv, *u = U + (size_t)t * dv;
        double *dqt = dq + t * ld_k, *dkt = dkk + t * ld_k, *dgt = dg + t * ld_k;
        double *dvt = dvv + t * ld_v;
        /* S'_t, as the forward formed it */
        for (int i = 0; i < dk; ++i) {
            const double a = exp((double)gt[i]);
            for (int j = 0; j < dv; ++j) Sp[(size_t)i * dv + j] = Sprev[(size_t)i * dv + j] * a;
        }
        /* o_t = S_t^T q_t */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] += (double)qt[i] * (double)dot[j];
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) acc += S[(size_t)i * dv + j] * (double)dot[j];
            dqt[i] = acc;
        }
        /* S_t = S'_t + k_t u_t^T */
        for (int j = 0; j < dv; ++j) du[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) du[j] += dS[(size_t)i * dv + j] * (double)kt[i];
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) acc += dS[(size_t)i * dv + j] * u[j];
            dkt[i] = acc;
        }
        /* u_t = beta_t (v_t - w_t) */
        double dbt = 0.0;
        for (int j = 0; j < dv; ++j) {
            dvt[j] = b * du[j];
            dbt += ((double)vt[j] - w[j]) * du[j];
        }
        db[t * ld_b] = dbt;
        /* w_t = S'_t^T k_t, with dw = -beta_t du (kept in du) */
        for (int j = 0; j < dv; ++j) du[j] = -b * du[j];
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] += (double)kt[i] * du[j];
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) acc += Sp[(size_t)i * dv + j] * du[j];
            dkt[i] += acc;
        }
        /* S'_t = Diag(exp(g_t)) S_{t-1} */
        for (int i = 0; i < dk; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) acc += dS[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];
            dgt[i] = acc;
            const double a = exp((double)gt[i]);
            for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] *= a;
        }
    }
    for (size_t e = 0; e < ss; ++e) dS0[e] = dS[e];
}

/* Packed varlen batch: inputs as in kda_oracle_fwd, dO [N, H, dv] fp32,
 * dST [n_seqs, H, dk, dv] fp32 or NULL (zeros).  Out (fp64): dq, dk, dg
 * [N, H, dk]; dv [N, H, dv]; dbeta [N, H]; dS0 [n_seqs, H, dk, dv].
 * Keeps every state of the longest sequence per thread.  Returns the number
 * of threads used, or -1 if the state buffer cannot be allocated.          */
int kda_oracle_vjp(const float *q, const float *k, const float *v,
                   const float *g, const float *beta, const float *S0,
                   const float *dO, const float *dST,
                   const int32_t *cu, int n_seqs, int H, int dk, int dv,
                   double *dq, double *dkk, double *dvv, double *dg, double *db,
                   double *dS0, int n_threads)
{
    int used = 1, failed = 0;
    int64_t Tmax = 0;
    for (int n = 0; n < n_seqs; ++n) {
        const int64_t T = (int64_t)cu[n + 1] - cu[n];
        if (T > Tmax) Tmax = T;
    }
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
    const int64_t pairs = (int64_t)n_seqs * H;
    const size_t ss = (size_t)dk * dv;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double *Sall = (double *)malloc(sizeof(double) * (size_t)(Tmax + 1) * ss);
        double *W = (double *)malloc(sizeof(double) * (size_t)(Tmax + 1) * dv);
        double *U = (double *)malloc(sizeof(double) * (size_t)(Tmax + 1) * dv);
        double *Sp = (double *)malloc(sizeof(double) * ss);
        double *dS = (double *)malloc(sizeof(double) * ss);
        double *du = (double *)malloc(sizeof(double) * (size_t)dv);
        const int ok = Sall && W && U && Sp && dS && du;
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < pairs; ++p) {
            if (!ok) continue;
            const int n = (int)(p / H), h = (int)(p % H);
            const int64_t t0 = cu[n], T = (int64_t)cu[n + 1] - cu[n];
            const size_t so = ((size_t)n * H + h) * ss;
            vjp_chain(T, dk, dv,
                      q + (t0 * H + h) * dk, k + (t0 * H + h) * dk,
                      v + (t0 * H + h) * dv, g + (t0 * H + h) * dk,
                      beta + t0 * H + h, dO + (t0 * H + h) * dv,
                      (int64_t)H * dk, (int64_t)H * dv, H,
                      S0 ? S0 + so : NULL, dST ? dST + so : NULL,
                      dq + (t0 * H + h) * dk, dkk + (t0 * H + h) * dk,
                      dvv + (t0 * H + h) * dv, dg + (t0 * H + h) * dk, db + t0 * H + h,
                      dS0 + so, Sall, W, U, Sp, dS, du);
        }
        free(Sall); free(W); free(U); free(Sp); free(dS); free(du);
    }
    return failed ? -1 : used;
}
