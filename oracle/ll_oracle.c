/*
 * fp64 oracle for log-linear attention in its Mamba-2 form.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links, includes or calls
 * this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline use it.  It is deliberately plain and slow: a direct evaluation of
 * the masked sum, one output row at a time, with no chunking, blocking,
 * fusion or reordering.
 *
 * Sources (cited by page title, language and section):
 *   [LLA-pt] "Log-Linear Attention" summary page, Portuguese
 *            (gist.science/pt/paper/2506.04761), §2 "Metodologia".
 *   [LLA-fr] "Log-Linear Attention" summary page, French
 *            (gist.science/fr/paper/2506.04761), §2 "Méthodologie".
 *
 * What is computed.  Attention is written O = (Q K^T ⊙ M_H) V with a
 * hierarchical mask M_H [LLA-fr §2 "Matrice de Masque Hiérarchique";
 * LLA-pt §2 "Máscara Hierárquica"].  The prefix before token t is cut into
 * Fenwick-tree buckets of sizes 1, 2, 4, 8, ... [LLA-pt §2 "Particionamento
 * Hierárquico"; LLA-fr §2 "Partitionnement par Arbre de Fenwick"], and each
 * level l carries a data-dependent weight lambda_t^(l) [LLA-fr §2, last
 * bullet of the mask paragraph].  The base model is Mamba-2 [LLA-pt §2
 * "Generalização"; LLA-fr §3 "Études de Cas"], whose mask is the
 * semiseparable decay mask.  Readings where the pages are silent:
 *   - decay and hierarchy compose:  M_H[t,s] = exp(sum_{r=s+1..t} a_r) *
 *     lambda_t[level(t,s)] for s <= t, 0 otherwise (a_0 never enters);
 *   - level(t,s) = 0 if s == t, else the bit length of (t XOR s), positions
 *     0-indexed; so level 0 is the token itself and level l >= 1 is the
 *     bucket of 2^(l-1) positions selected by bit l-1 of t;
 *   - no softmax, no normalisation, no 1/sqrt(d) scaling, identity features.
 *
 * So, for every (b, h, t):
 *   o[t,:] = sum_{s=0..t} exp(sum_{r=s+1..t} a[r]) * lambda[t, level(t,s)]
 *                         * (sum_d q[t,d] k[s,d]) * v[s,:]
 *
 * Everything is fp64; exp is the host libm exp.  The decay exponent is summed
 * directly over (s, t] while walking s downwards, so no large prefix sums are
 * subtracted.
 *
 * Layouts (all row-major, contiguous, fp64):
 *   q, k [BH, T, dk]; v [BH, T, dv]; a [BH, T]; lam [BH, T, L]; out [n, dv].
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stddef.h>

/* Fenwick level of key s as seen from query t (both 0-indexed, s <= t). */
int ll_oracle_level(int64_t t, int64_t s)
{
    if (s == t)
        return 0;
    uint64_t x = (uint64_t)t ^ (uint64_t)s;
    int bits = 0;
    while (x != 0) {
        bits += 1;
        x >>= 1;
    }
    return bits;
}

/* One output row o[t,:] for head bh.  Returns 0, or -1 if a level does not
 * fit in L (the caller's lambda is too narrow). */
static int oracle_row(const double *q, const double *k, const double *v,
                      const double *a, const double *lam,
                      int64_t T, int64_t dk, int64_t dv, int64_t L,
                      int64_t bh, int64_t t, double *o)
{
    const double *qt = q + (bh * T + t) * dk;
    const double *lt = lam + (bh * T + t) * L;
    const double *ah = a + bh * T;
    for (int64_t e = 0; e < dv; ++e)
        o[e] = 0.0;
    double logdecay = 0.0; /* sum of a over (s, t] */
    for (int64_t s = t; s >= 0; --s) {
        if (s < t)
            logdecay += ah[s + 1];
        int lev = ll_oracle_level(t, s);
        if (lev >= L)
            return -1;
        const double *ks = k + (bh * T + s) * dk;
        const double *vs = v + (bh * T + s) * dv;
        double score = 0.0;
        for (int64_t d = 0; d < dk; ++d)
            score += qt[d] * ks[d];
        double w = exp(logdecay) * lt[lev] * score;
        for (int64_t e = 0; e < dv; ++e)
            o[e] += w * vs[e];
    }
    return 0;
}

/* Evaluate the rows listed in rows[2*i] = bh, rows[2*i+1] = t into
 * out[i, :].  Rows are independent; OpenMP spreads them over the host's
 * cores.  Returns 0, -1 for a level beyond L, -2 for a row out of range. */
int ll_oracle_fwd_rows(const double *q, const double *k, const double *v,
                       const double *a, const double *lam,
                       int64_t BH, int64_t T, int64_t dk, int64_t dv, int64_t L,
                       int64_t nrows, const int64_t *rows, double *out)
{
    int status = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t bh = rows[2 * i], t = rows[2 * i + 1];
        int rc;
        if (bh < 0 || bh >= BH || t < 0 || t >= T)
            rc = -2;
        else
            rc = oracle_row(q, k, v, a, lam, T, dk, dv, L, bh, t, out + i * dv);
        if (rc != 0) {
#pragma omp critical
            status = rc;
        }
    }
    return status;
}

/* Every row of every head: out [BH, T, dv]. */
int ll_oracle_fwd(const double *q, const double *k, const double *v,
                  const double *a, const double *lam,
                  int64_t BH, int64_t T, int64_t dk, int64_t dv, int64_t L,
                  double *out)
{
    int status = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int64_t bh = 0; bh < BH; ++bh) {
        for (int64_t t = 0; t < T; ++t) {
            int rc = oracle_row(q, k, v, a, lam, T, dk, dv, L, bh, t,
                                out + (bh * T + t) * dv);
            if (rc != 0) {
#pragma omp critical
                status = rc;
            }
        }
    }
    return status;
}

/* Number of threads OpenMP will use (reported with the CPU baseline). */
int ll_oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
