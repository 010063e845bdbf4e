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
 *
 * The backward section further down differentiates the same sum.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>

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

/* ---- backward --------------------------------------------------------------
 *
 * Gradients of the scalar sum_t do[t,:] . o[t,:] with respect to every input,
 * by differentiating the definition above term by term.  With
 *   w(t,s) = exp(sum_{r=s+1..t} a_r) * lambda[t, level(t,s)]   (s <= t)
 *   P(t,s) = w(t,s) * (q_t . k_s) * (do_t . v_s):
 *   dq_t           = sum_{s<=t} w(t,s) (do_t . v_s) k_s
 *   dk_s           = sum_{t>=s} w(t,s) (do_t . v_s) q_t
 *   dv_s           = sum_{t>=s} w(t,s) (q_t . k_s) do_t
 *   dlambda_t[l]   = sum_{s<=t, level(t,s)=l} exp(sum_{r=s+1..t} a_r) (q_t . k_s)(do_t . v_s)
 *   da_r (r >= 1)  = sum_{t>=r} sum_{s<r} P(t,s)     (a_r sits in the decay of
 *                    exactly the pairs s < r <= t); da_0 = 0 (a_0 never enters)
 * The last one is evaluated as da_r = sum_{t>=r} (Pq_t - Pk_t) with
 * Pq_t = sum_{s<=t} P(t,s) and Pk_t = sum_{t'>=t} P(t',t): the pairs with
 * s >= r cancel between the two sums.  Backpropagation through the
 * per-level weights lambda is the part the French page names as needing
 * custom kernels ([LLA-fr §5 "Signification et Limites", limits list]).
 *
 * Layouts: do [BH, T, dv]; dq, dk [BH, T, dk]; dv [BH, T, dv]; da [BH, T];
 * dlam [BH, T, L].
 */

/* Query-side row t of head bh: dq_t, dlam_t and Pq_t. */
static int oracle_bwd_qrow(const double *q, const double *k, const double *v, const double *a,
                           const double *lam, const double *dout, int64_t T, int64_t dk, int64_t dv,
                           int64_t L, int64_t bh, int64_t t, double *dq, double *dlam, double *pq)
{
    const double *qt = q + (bh * T + t) * dk;
    const double *dot = dout + (bh * T + t) * dv;
    const double *lt = lam + (bh * T + t) * L;
    const double *ah = a + bh * T;
    for (int64_t d = 0; d < dk; ++d)
        dq[d] = 0.0;
    for (int64_t l = 0; l < L; ++l)
        dlam[l] = 0.0;
    double psum = 0.0, logdecay = 0.0;
    for (int64_t s = t; s >= 0; --s) {
        if (s < t)
            logdecay += ah[s + 1];
        int lev = ll_oracle_level(t, s);
        if (lev >= L)
            return -1;
        const double *ks = k + (bh * T + s) * dk;
        const double *vs = v + (bh * T + s) * dv;
        double qk = 0.0, dov = 0.0;
        for (int64_t d = 0; d < dk; ++d)
            qk += qt[d] * ks[d];
        for (int64_t e = 0; e < dv; ++e)
            dov += dot[e] * vs[e];
        double dec = exp(logdecay);
        double w = dec * lt[lev];
        for (int64_t d = 0; d < dk; ++d)
            dq[d] += w * dov * ks[d];
        dlam[lev] += dec * qk * dov;
        psum += w * qk * dov;
    }
    *pq = psum;
    return 0;
}

/* Key-side row s of head bh: dk_s, dv_s and Pk_s. */
static int oracle_bwd_krow(const double *q, const double *k, const double *v, const double *a,
                           const double *lam, const double *dout, int64_t T, int64_t dk, int64_t dv,
                           int64_t L, int64_t bh, int64_t s, double *dks, double *dvs, double *pk)
{
    const double *ks = k + (bh * T + s) * dk;
    const double *vs = v + (bh * T + s) * dv;
    const double *ah = a + bh * T;
    for (int64_t d = 0; d < dk; ++d)
        dks[d] = 0.0;
    for (int64_t e = 0; e < dv; ++e)
        dvs[e] = 0.0;
    double psum = 0.0, logdecay = 0.0;
    for (int64_t t = s; t < T; ++t) {
        if (t > s)
            logdecay += ah[t];
        int lev = ll_oracle_level(t, s);
        if (lev >= L)
            return -1;
        const double *qt = q + (bh * T + t) * dk;
        const double *dot = dout + (bh * T + t) * dv;
        double qk = 0.0, dov = 0.0;
        for (int64_t d = 0; d < dk; ++d)
            qk += qt[d] * ks[d];
        for (int64_t e = 0; e < dv; ++e)
            dov += dot[e] * vs[e];
        double w = exp(logdecay) * lam[(bh * T + t) * L + lev];
        for (int64_t d = 0; d < dk; ++d)
            dks[d] += w * dov * qt[d];
        for (int64_t e = 0; e < dv; ++e)
            dvs[e] += w * qk * dot[e];
        psum += w * qk * dov;
    }
    *pk = psum;
    return 0;
}

/* Every gradient of every head. */
int ll_oracle_bwd(const double *q, const double *k, const double *v, const double *a, const double *lam,
                  const double *dout, int64_t BH, int64_t T, int64_t dk, int64_t dv, int64_t L, double *dq,
                  double *dkk, double *dvv, double *da, double *dlam)
{
    int status = 0;
    double *pq = (double *)calloc((size_t)(BH * T > 0 ? BH * T : 1), sizeof(double));
    double *pk = (double *)calloc((size_t)(BH * T > 0 ? BH * T : 1), sizeof(double));
    if (!pq || !pk) {
        free(pq);
        free(pk);
        return -3;
    }
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int64_t bh = 0; bh < BH; ++bh) {
        for (int64_t t = 0; t < T; ++t) {
            int rc = oracle_bwd_qrow(q, k, v, a, lam, dout, T, dk, dv, L, bh, t, dq + (bh * T + t) * dk,
                                     dlam + (bh * T + t) * L, pq + bh * T + t);
            if (rc == 0)
                rc = oracle_bwd_krow(q, k, v, a, lam, dout, T, dk, dv, L, bh, t, dkk + (bh * T + t) * dk,
                                     dvv + (bh * T + t) * dv, pk + bh * T + t);
            if (rc != 0) {
#pragma omp critical
                status = rc;
            }
        }
    }
    for (int64_t bh = 0; bh < BH; ++bh) {
        double run = 0.0;
        for (int64_t r = T - 1; r >= 1; --r) {
            run += pq[bh * T + r] - pk[bh * T + r];
            da[bh * T + r] = run;
        }
        if (T > 0)
            da[bh * T] = 0.0;
    }
    free(pq);
    free(pk);
    return status;
}

/* Selected query-side rows (rows[2i] = bh, rows[2i+1] = t): dq [n, dk],
 * dlam [n, L]. */
int ll_oracle_bwd_qrows(const double *q, const double *k, const double *v, const double *a, const double *lam,
                        const double *dout, int64_t BH, int64_t T, int64_t dk, int64_t dv, int64_t L,
                        int64_t nrows, const int64_t *rows, double *dq, double *dlam)
{
    int status = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t bh = rows[2 * i], t = rows[2 * i + 1];
        double pq;
        int rc = (bh < 0 || bh >= BH || t < 0 || t >= T)
                     ? -2
                     : oracle_bwd_qrow(q, k, v, a, lam, dout, T, dk, dv, L, bh, t, dq + i * dk, dlam + i * L, &pq);
        if (rc != 0) {
#pragma omp critical
            status = rc;
        }
    }
    return status;
}

/* Selected key-side rows (rows[2i] = bh, rows[2i+1] = s): dk [n, dk],
 * dv [n, dv]. */
int ll_oracle_bwd_krows(const double *q, const double *k, const double *v, const double *a, const double *lam,
                        const double *dout, int64_t BH, int64_t T, int64_t dk, int64_t dv, int64_t L,
                        int64_t nrows, const int64_t *rows, double *dkk, double *dvv)
{
    int status = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t bh = rows[2 * i], s = rows[2 * i + 1];
        double pk;
        int rc = (bh < 0 || bh >= BH || s < 0 || s >= T)
                     ? -2
                     : oracle_bwd_krow(q, k, v, a, lam, dout, T, dk, dv, L, bh, s, dkk + i * dk, dvv + i * dv, &pk);
        if (rc != 0) {
#pragma omp critical
            status = rc;
        }
    }
    return status;
}

/* da at selected positions from the pairs within W tokens of r:
 * sum over s in [max(0, r-W), r) and t in [r, min(T, r+W)) of P(t,s), at
 * the pairs' absolute positions (levels depend on them).  With W >= T this
 * is the exact da_r; for long sequences the omitted pairs carry a decay of
 * at least W consecutive a's, which the caller bounds.  rows[2i] = bh,
 * rows[2i+1] = r (r >= 1). */
int ll_oracle_da_window(const double *q, const double *k, const double *v, const double *a, const double *lam,
                        const double *dout, int64_t BH, int64_t T, int64_t dk, int64_t dv, int64_t L,
                        int64_t nrows, const int64_t *rows, int64_t W, double *out)
{
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
        const int64_t bh = rows[2 * i], r = rows[2 * i + 1];
        if (bh < 0 || bh >= BH || r < 1 || r >= T) {
#pragma omp critical
            status = -2;
            continue;
        }
        const double *ah = a + bh * T;
        const int64_t s0 = r - W > 0 ? r - W : 0, t1 = r + W < T ? r + W : T;
        double total = 0.0;
        for (int64_t t = r; t < t1; ++t) {
            const double *qt = q + (bh * T + t) * dk;
            const double *dot = dout + (bh * T + t) * dv;
            double logdecay = 0.0; /* sum of a over (s, t] */
            for (int64_t rr = r; rr <= t; ++rr)
                logdecay += ah[rr];
            for (int64_t s = r - 1; s >= s0; --s) {
                if (s < r - 1)
                    logdecay += ah[s + 1];
                const int lev = ll_oracle_level(t, s);
                if (lev >= L) {
#pragma omp critical
                    status = -1;
                    break;
                }
                const double *ks = k + (bh * T + s) * dk;
                const double *vs = v + (bh * T + s) * dv;
                double qk = 0.0, dov = 0.0;
                for (int64_t d = 0; d < dk; ++d)
                    qk += qt[d] * ks[d];
                for (int64_t e = 0; e < dv; ++e)
                    dov += dot[e] * vs[e];
                total += exp(logdecay) * lam[(bh * T + t) * L + lev] * qk * dov;
            }
        }
        out[i] = total;
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
