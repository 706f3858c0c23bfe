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

/* ---------------------------------------------------------------------------
 * Backward pass (reverse-mode adjoint of the recurrence above).
 *
 * Gradients are what a training step needs: "Hybrid Attention"
 * (kimi-k3.adriaflores.com), section "But isn't a recurrent update
 * sequential?", checks the chunkwise form's outputs and gradients against the
 * token recurrence, which is the function differentiated here (the four steps
 * above).  With a scalar loss whose gradients with respect to the
 * outputs o_t and the final states are given (dO, dS_T), each token's four
 * steps are differentiated in reverse order:
 *
 *   forward (from S_prev):  D = Diag(exp g) S_prev;  p = D^T k;  r = v - p;
 *                           S = D + beta k r^T;      o = scale S^T q
 *   reverse (dS = gradient with respect to S, from later tokens):
 *     4. read:    dS += scale q do^T;             dq = scale S do
 *     3. correct: w = dS^T k;  dr = beta w;  dbeta = r . w;  dk = beta dS r;
 *                 dD = dS  (the direct path)
 *     2. predict: dv = dr;  dp = -dr;  dD += k dp^T;  dk += D dp
 *     1. fade:    dg_i = sum_j D_ij dD_ij  (alpha_i * dalpha_i, as D = alpha S_prev);
 *                 dS_prev = Diag(exp g) dD
 *
 * The state before each token is needed in reverse order.  A forward pass
 * stores the state at the start of every segment of seg_len tokens; each
 * segment is then recomputed from its stored state (the same token function,
 * so the values are exactly those of a pass that stored every state) and
 * walked backwards.
 * ------------------------------------------------------------------------- */

/* Reverse of one token.  S_prev is the state before the token; dS holds the
 * gradient with respect to the state after it and is replaced by the
 * gradient with respect to S_prev.  work holds 2 dk dv + 3 dv doubles. */
static void oracle_token_backward(const double *S_prev, double *dS, int64_t dk, int64_t dv,
                                  const double *q, const double *k, const double *v,
                                  const double *g, double beta, double scale,
                                  const double *dout, double *dq, double *dkey,
                                  double *dval, double *dg, double *dbeta,
                                  double *work)
{
    double *D = work, *S = work + dk * dv, *r = work + 2 * dk * dv;
    double *w = r + dv, *dp = w + dv;
    double acc;
    int64_t i, j;
    /* Recompute the token's forward values. */
    for (i = 0; i < dk; ++i) {
        const double alpha = exp(g[i]);
        for (j = 0; j < dv; ++j) D[i * dv + j] = alpha * S_prev[i * dv + j];
    }
    for (j = 0; j < dv; ++j) {
        acc = 0.0;
        for (i = 0; i < dk; ++i) acc += D[i * dv + j] * k[i];
        r[j] = v[j] - acc;
    }
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j) S[i * dv + j] = D[i * dv + j] + beta * k[i] * r[j];
    /* Reverse of the read (o = scale S^T q). */
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j) dS[i * dv + j] += scale * q[i] * dout[j];
    for (i = 0; i < dk; ++i) {
        acc = 0.0;
        for (j = 0; j < dv; ++j) acc += S[i * dv + j] * dout[j];
        dq[i] = scale * acc;
    }
    /* Reverse of the correction (S = D + beta k r^T). */
    for (j = 0; j < dv; ++j) {
        acc = 0.0;
        for (i = 0; i < dk; ++i) acc += k[i] * dS[i * dv + j];
        w[j] = acc;
    }
    acc = 0.0;
    for (j = 0; j < dv; ++j) acc += r[j] * w[j];
    *dbeta = acc;
    for (i = 0; i < dk; ++i) {
        acc = 0.0;
        for (j = 0; j < dv; ++j) acc += dS[i * dv + j] * r[j];
        dkey[i] = beta * acc;
    }
    /* Reverse of the prediction (r = v - D^T k). */
    for (j = 0; j < dv; ++j) {
        dval[j] = beta * w[j];
        dp[j] = -beta * w[j];
    }
    for (i = 0; i < dk; ++i) {
        acc = 0.0;
        for (j = 0; j < dv; ++j) acc += D[i * dv + j] * dp[j];
        dkey[i] += acc;
    }
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j) dS[i * dv + j] += k[i] * dp[j];   /* dS is now dD */
    /* Reverse of the fade (D = Diag(exp g) S_prev). */
    for (i = 0; i < dk; ++i) {
        const double alpha = exp(g[i]);
        acc = 0.0;
        for (j = 0; j < dv; ++j) acc += D[i * dv + j] * dS[i * dv + j];
        dg[i] = acc;
        for (j = 0; j < dv; ++j) dS[i * dv + j] *= alpha;
    }
}

int kda_oracle_prefill_backward_f64(int64_t num_seqs, const int64_t *cu, int64_t H,
                                    int64_t dk, int64_t dv, double scale,
                                    const double *q, const double *k, const double *v,
                                    const double *g, const double *beta,
                                    const double *S0, const double *dO,
                                    const double *dS_T, double *dq, double *dkey,
                                    double *dval, double *dg, double *dbeta,
                                    double *dS0, int64_t seg_len, int nthreads)
{
    int64_t unit, units;
    int err = 0;
    if (num_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu) return -1;
    if (check_cu(num_seqs, cu)) return -2;
    if (cu[num_seqs] > 0 && (!q || !k || !v || !g || !beta || !dO || !dq || !dkey || !dval || !dg || !dbeta))
        return -1;
    if (seg_len <= 0) seg_len = 64;
    units = num_seqs * H;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (unit = 0; unit < units; ++unit) {
        const int64_t n = unit / H, h = unit % H, a0 = cu[n], L = cu[n + 1] - cu[n];
        const int64_t nseg = (L + seg_len - 1) / seg_len, sz = dk * dv;
        /* segment-start states, the states inside one segment, dS, work */
        double *buf = (double *)malloc((size_t)((nseg + seg_len + 4) * sz + 3 * dv) * sizeof(double));
        double *ck, *seg, *dS, *work;
        int64_t t, m;
        if (!buf) { err |= 1; continue; }
        ck = buf;
        seg = ck + nseg * sz;
        dS = seg + seg_len * sz;
        work = dS + sz;
        /* forward: remember the state at every segment start */
        if (S0) memcpy(dS, S0 + unit * sz, (size_t)sz * sizeof(double));
        else memset(dS, 0, (size_t)sz * sizeof(double));
        for (t = 0; t < L; ++t) {
            const int64_t th = (a0 + t) * H + h;
            if (t % seg_len == 0) memcpy(ck + (t / seg_len) * sz, dS, (size_t)sz * sizeof(double));
            oracle_token(dS, dk, dv, q + th * dk, k + th * dk, v + th * dv, g + th * dk, beta[th],
                         scale, 1, NULL, work);
        }
        /* backward, last segment first */
        if (dS_T) memcpy(dS, dS_T + unit * sz, (size_t)sz * sizeof(double));
        else memset(dS, 0, (size_t)sz * sizeof(double));
        for (m = nseg - 1; m >= 0; --m) {
            const int64_t s0 = m * seg_len, s1 = (s0 + seg_len < L) ? s0 + seg_len : L;
            memcpy(seg, ck + m * sz, (size_t)sz * sizeof(double));
            for (t = s0 + 1; t < s1; ++t) {
                const int64_t th = (a0 + t - 1) * H + h;
                double *Sn = seg + (t - s0) * sz;
                memcpy(Sn, Sn - sz, (size_t)sz * sizeof(double));
                oracle_token(Sn, dk, dv, q + th * dk, k + th * dk, v + th * dv, g + th * dk, beta[th],
                             scale, 1, NULL, work);
            }
            for (t = s1 - 1; t >= s0; --t) {
                const int64_t th = (a0 + t) * H + h;
                oracle_token_backward(seg + (t - s0) * sz, dS, dk, dv, q + th * dk, k + th * dk,
                                      v + th * dv, g + th * dk, beta[th], scale, dO + th * dv,
                                      dq + th * dk, dkey + th * dk, dval + th * dv, dg + th * dk,
                                      dbeta + th, work);
            }
        }
        if (dS0) memcpy(dS0 + unit * sz, dS, (size_t)sz * sizeof(double));
        free(buf);
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
