/*
 * kda_oracle.c -- CPU fp64 oracle for the Kimi Delta Attention (KDA) core.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition the GPU path is checked against.  Only tests/, the smoke check
 * in __graft_entry__.py and the cpu_baseline leg of bench.py may load it.
 * It shares no code, header, table or helper with the HIP library, and the
 * HIP library never calls it.
 *
 * What it computes (per sequence n, per head h, tokens in order):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *   o_t = scale * S_t^T q_t,        alpha_t = exp(g_t)  (one factor per key channel)
 *
 * Sources:
 *   - "Understanding Kimi K3's attention" (dhruvpendharkar.github.io): the
 *     symbol table (S is d_k x d_v, alpha_t = exp(g_t) is a per-key-channel
 *     retention vector, beta_t a scalar write strength), the full state-update
 *     equation, the readout equation, and the equivalent rewritten update in
 *     which the decayed state's prediction (Diag(alpha_t) S_{t-1})^T k_t is
 *     subtracted from v_t.
 *   - "Hybrid Attention" (kimi-k3.adriaflores.com), section "KDA: don't write
 *     the same information twice": the per-token order retain -> predict ->
 *     correct, on a state indexed [key channel][value channel].
 *   - "KDA: the memory matrix" (kimi-k3-course.pages.dev, lesson 2): the
 *     readout uses S_t, i.e. the state after the token's own write.
 *   - "Kimi K3.1 and the Road From Softmax Attention to KDA"
 *     (neuralmasteryai.com), section 5: the same update and readout.
 *
 * The expansion used below is the rewritten form, term for term:
 *   1. fade:    D = Diag(exp g_t) S_{t-1}        (scales ROWS = key channels)
 *   2. predict: p = D^T k_t                       (skipped, p = 0, if !delta)
 *   3. correct: S_t = D + beta_t k_t (v_t - p)^T
 *   4. read:    o_t = scale * S_t^T q_t
 * Expanding (I - beta k k^T) D + beta k v^T = D + beta k (v - D^T k)^T shows
 * this is the product form exactly.  With delta == 0 the update is the plain
 * gated linear-attention write S_t = D + beta_t k_t v_t^T; with g = 0 and
 * beta = 1 that is linear attention (neuralmasteryai.com, section 2).
 *
 * Readings where the pages are silent (listed in the design notes):
 *   - scale multiplies the readout; scale = 1 gives o_t = S_t^T q_t exactly.
 *   - variable-length batches: the state restarts at every sequence start,
 *     from S0[n,h] when S0 is given and from zeros otherwise.  An empty
 *     sequence returns its initial state unchanged.
 *
 * Layouts (row-major, contiguous, host memory):
 *   q, k, g : [T_total, H, dk]     v, o : [T_total, H, dv]    beta : [T_total, H]
 *   S0, S   : [N, H, dk, dv]       cu   : [N + 1], cu[0] = 0, non-decreasing
 *
 * All arithmetic is IEEE double, sums in plain index order, no fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "kda_oracle.h"

int kda_oracle_version(void) { return 1; }

/* One token of the recurrence on one (n, h) state S[dk][dv], in place.
 * tmp holds dv doubles.  o may be NULL (no readout requested). */
static void oracle_token(double *S, int64_t dk, int64_t dv,
                         const double *q, const double *k, const double *v,
                         const double *g, double beta, double scale, int delta,
                         double *o, double *tmp)
{
    int64_t i, j;
    /* 1. fade: Diag(alpha_t) acts on the key-channel rows. */
    for (i = 0; i < dk; ++i) {
        const double a = exp(g[i]);
        double *row = S + i * dv;
        for (j = 0; j < dv; ++j) row[j] *= a;
    }
    /* 2. predict what the decayed memory returns for k_t. */
    for (j = 0; j < dv; ++j) tmp[j] = 0.0;
    if (delta) {
        for (i = 0; i < dk; ++i) {
            const double ki = k[i];
            const double *row = S + i * dv;
            for (j = 0; j < dv; ++j) tmp[j] += row[j] * ki;
        }
    }
    /* 3. correct: write the residual v_t - prediction along k_t, strength beta_t. */
    for (j = 0; j < dv; ++j) tmp[j] = v[j] - tmp[j];
    for (i = 0; i < dk; ++i) {
        const double bk = beta * k[i];
        double *row = S + i * dv;
        for (j = 0; j < dv; ++j) row[j] += bk * tmp[j];
    }
    /* 4. read the state after this token's write. */
    if (o) {
        for (j = 0; j < dv; ++j) tmp[j] = 0.0;
        for (i = 0; i < dk; ++i) {
            const double qi = q[i];
            const double *row = S + i * dv;
            for (j = 0; j < dv; ++j) tmp[j] += row[j] * qi;
        }
        for (j = 0; j < dv; ++j) o[j] = scale * tmp[j];
    }
}

static int check_cu(int64_t num_seqs, const int64_t *cu)
{
    int64_t n;
    if (cu[0] != 0) return -2;
    for (n = 0; n < num_seqs; ++n)
        if (cu[n + 1] < cu[n]) return -2;
    return 0;
}

int kda_oracle_prefill_f64(int64_t num_seqs, const int64_t *cu, int64_t H,
                           int64_t dk, int64_t dv, double scale, int delta,
                           const double *q, const double *k, const double *v,
                           const double *g, const double *beta,
                           const double *S0, double *o, double *S_out,
                           int nthreads)
{
    int64_t unit, units;
    int err = 0;
    if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu) return -1;
    if (check_cu(num_seqs, cu)) return -2;
    if (cu[num_seqs] > 0 && (!q || !k || !v || !g || !beta || !o)) return -1;
    units = num_seqs * H;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (unit = 0; unit < units; ++unit) {
        const int64_t n = unit / H, h = unit % H;
        double *S = (double *)malloc((size_t)(dk * dv + dv) * sizeof(double));
        double *tmp;
        int64_t t;
        if (!S) { err |= 1; continue; }
        tmp = S + dk * dv;
        if (S0) memcpy(S, S0 + unit * dk * dv, (size_t)(dk * dv) * sizeof(double));
        else memset(S, 0, (size_t)(dk * dv) * sizeof(double));
        for (t = cu[n]; t < cu[n + 1]; ++t) {
            const int64_t th = t * H + h;
            oracle_token(S, dk, dv, q + th * dk, k + th * dk, v + th * dv,
                         g + th * dk, beta[th], scale, delta, o + th * dv, tmp);
        }
        if (S_out) memcpy(S_out + unit * dk * dv, S, (size_t)(dk * dv) * sizeof(double));
        free(S);
    }
    return err ? -3 : 0;
}

int kda_oracle_decode_step_f64(int64_t N, int64_t H, int64_t dk, int64_t dv,
                               double scale, const double *q, const double *k,
                               const double *v, const double *g,
                               const double *beta, double *S, double *o,
                               int nthreads)
{
    int64_t unit, units;
    int err = 0;
    if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (N > 0 && (!q || !k || !v || !g || !beta || !S || !o)) return -1;
    units = N * H;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel for schedule(static) reduction(| : err)
    for (unit = 0; unit < units; ++unit) {
        double *tmp = (double *)malloc((size_t)dv * sizeof(double));
        if (!tmp) { err |= 1; continue; }
        oracle_token(S + unit * dk * dv, dk, dv, q + unit * dk, k + unit * dk,
                     v + unit * dv, g + unit * dk, beta[unit], scale, 1,
                     o + unit * dv, tmp);
        free(tmp);
    }
    return err ? -3 : 0;
}

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
