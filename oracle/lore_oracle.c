/*
 * fp64 reference for LORE-KV's projected deletion score.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the bench's CPU
 * baseline load this file's shared object; the HIP library neither links nor
 * calls it, and it shares no code, header or table with the HIP path.
 *
 * What it computes follows the LORE-KV project page ("Monte Carlo Estimation
 * for KV-Cache Eviction"), section "Projected deletion score", Eqs. 5-7:
 *
 *   a_{q,i}  attention probability of scoring query q on cached token i,
 *   o_q      = sum_i a_{q,i} v_i, the attention output,
 *   e_{q,i}  = a_{q,i} / (1 - a_{q,i} + eps) * || W_O (v_i - o_q) ||,
 *   S_i      = psi(E_{i,W}) + lambda_L * sum_m omega_m psi(E_{i,m}),
 *
 * with psi the arithmetic mean over the query set it is applied to.  The norm
 * through the head's output projection W_h (a d_model x d column slice of
 * W_O) is taken through an upper-triangular R_h with R_h^T R_h = W_h^T W_h,
 * so that ||W_h x|| = ||R_h x|| exactly; the caller passes R_h (a Cholesky
 * factor) and the difference v_i - o_q is formed directly, without expanding
 * the square.
 *
 * Query rows: rows 0..w-1 are the prompt window (the last w prompt positions,
 * "Prefill" in the page's Method section); row r sits at position n-w+r and,
 * as in the causal prefill that produced it, sees tokens 0..n-w+r.  Rows
 * w + m*T + t are lookahead query t of trajectory m (Eq. 1) and see all n
 * prompt tokens.  Softmax logits are q.k / sqrt(d).
 *
 * Layouts (row-major, fp64):
 *   Q [batch][h_q][n_q][d], K and V [batch][h_kv][n][d],
 *   R [h_q][d][d], omega [batch][m_traj],
 *   row_max, row_sum [batch][h_q][n_q]   (max of q.k/sqrt(d); sum of exp(s-max)),
 *   O [batch][h_q][n_q][d],
 *   S_head [batch][h_q][n] (per query head, before the GQA group mean).
 * Query head h reads KV head h / (h_q / h_kv).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Last token index that scoring row r may attend to. */
static long visible_last(int r, int n, int w)
{
    return r < w ? (long)n - w + r : (long)n - 1;
}

static double dot(const double *a, const double *b, int d)
{
    double s = 0.0;
    for (int k = 0; k < d; ++k) s += a[k] * b[k];
    return s;
}

/* Softmax statistics and attention output of every scoring row. */
int ora_lore_attention(int batch, int n, int h_q, int h_kv, int d, int n_q, int w,
                       const double *Q, const double *K, const double *V,
                       double *row_max, double *row_sum, double *O, int nthreads)
{
    if (h_kv <= 0 || h_q % h_kv != 0 || n < w || n <= 0 || d <= 0) return 1;
    const int G = h_q / h_kv;
    const double scale = 1.0 / sqrt((double)d);
    const long rows = (long)batch * h_q * n_q;
    /* threads for this call only (a num_threads clause, not the process-wide
     * setting, so a call with nthreads = 1 leaves later calls on all cores) */
#ifdef _OPENMP
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#endif
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (long row = 0; row < rows; ++row) {
        const int r = (int)(row % n_q);
        const int h = (int)((row / n_q) % h_q);
        const int b = (int)(row / ((long)n_q * h_q));
        const int g = h / G;
        const double *q = Q + row * d;
        const double *Kg = K + ((long)b * h_kv + g) * n * d;
        const double *Vg = V + ((long)b * h_kv + g) * n * d;
        const long last = visible_last(r, n, w);
        double m = -INFINITY;
        for (long i = 0; i <= last; ++i) {
            double s = dot(q, Kg + i * d, d) * scale;
            if (s > m) m = s;
        }
        double l = 0.0;
        double *o = O + row * d;
        for (int k = 0; k < d; ++k) o[k] = 0.0;
        for (long i = 0; i <= last; ++i) {
            double p = exp(dot(q, Kg + i * d, d) * scale - m);
            l += p;
            for (int k = 0; k < d; ++k) o[k] += p * Vg[i * d + k];
        }
        for (int k = 0; k < d; ++k) o[k] /= l;
        row_max[row] = m;
        row_sum[row] = l;
    }
    return 0;
}

/* Per-query-head aggregated deletion score S_head[b][h][i] for every token.
 * row_max, row_sum and O must come from ora_lore_attention on the same inputs. */
int ora_lore_scores(int batch, int n, int h_q, int h_kv, int d, int w, int m_traj, int t_len,
                    double eps, double lambda_l,
                    const double *Q, const double *K, const double *V, const double *R,
                    const double *omega, const double *row_max, const double *row_sum,
                    const double *O, double *S_head, int nthreads)
{
    if (h_kv <= 0 || h_q % h_kv != 0 || n < w || n <= 0 || d <= 0 || m_traj < 0 || t_len < 0)
        return 1;
    if (m_traj > 0 && t_len == 0) return 1;
    const int G = h_q / h_kv;
    const int n_q = w + m_traj * t_len;
    const double scale = 1.0 / sqrt((double)d);
#ifdef _OPENMP
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#endif
    double *ot = (double *)malloc(sizeof(double) * (size_t)n_q * d);
    if (!ot) return 2;
    for (int b = 0; b < batch; ++b) {
        for (int h = 0; h < h_q; ++h) {
            const int g = h / G;
            const double *Rh = R + (long)h * d * d;
            const double *Qh = Q + ((long)b * h_q + h) * n_q * d;
            const double *Kg = K + ((long)b * h_kv + g) * n * d;
            const double *Vg = V + ((long)b * h_kv + g) * n * d;
            const double *mh = row_max + ((long)b * h_q + h) * n_q;
            const double *lh = row_sum + ((long)b * h_q + h) * n_q;
            const double *Oh = O + ((long)b * h_q + h) * n_q * d;
            const double *om = omega + (long)b * m_traj;
            double *Sh = S_head + ((long)b * h_q + h) * n;
            /* R_h o_q for every row */
            for (int r = 0; r < n_q; ++r)
                for (int k = 0; k < d; ++k) {
                    double s = 0.0;
                    for (int j = k; j < d; ++j) s += Rh[k * d + j] * Oh[r * d + j];
                    ot[r * d + k] = s;
                }
#pragma omp parallel num_threads(nt)
            {
                double *vt = (double *)malloc(sizeof(double) * (size_t)d);
                double *psi_m = (double *)malloc(sizeof(double) * (size_t)(m_traj > 0 ? m_traj : 1));
#pragma omp for schedule(static)
                for (long i = 0; i < n; ++i) {
                    const double *vi = Vg + i * d;
                    for (int k = 0; k < d; ++k) {
                        double s = 0.0;
                        for (int j = k; j < d; ++j) s += Rh[k * d + j] * vi[j];
                        vt[k] = s;
                    }
                    double psi_w = 0.0;
                    for (int mm = 0; mm < m_traj; ++mm) psi_m[mm] = 0.0;
                    for (int r = 0; r < n_q; ++r) {
                        double e = 0.0;
                        if (i <= visible_last(r, n, w)) {
                            double s = dot(Qh + r * d, Kg + i * d, d) * scale;
                            double a = exp(s - mh[r]) / lh[r];
                            double nrm = 0.0;
                            for (int k = 0; k < d; ++k) {
                                double diff = vt[k] - ot[r * d + k];
                                nrm += diff * diff;
                            }
                            e = a / (1.0 - a + eps) * sqrt(nrm);
                        }
                        if (r < w) psi_w += e;
                        else psi_m[(r - w) / t_len] += e;
                    }
                    double S = (w > 0) ? psi_w / w : 0.0;
                    for (int mm = 0; mm < m_traj; ++mm)
                        S += lambda_l * om[mm] * (psi_m[mm] / t_len);
                    Sh[i] = S;
                }
                free(vt);
                free(psi_m);
            }
        }
    }
    free(ot);
    return 0;
}

int ora_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
