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
 * OpenMP iteration.
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
