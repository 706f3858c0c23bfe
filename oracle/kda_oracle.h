/*
 * kda_oracle.h -- CPU fp64 oracle for the KDA core (TEST INFRASTRUCTURE ONLY).
 *
 * Used only by tests/, the smoke check and bench.py's cpu_baseline leg.  The
 * HIP library never includes this header.  Semantics are documented in
 * kda_oracle.c.  Every function returns 0 on success and a negative value on
 * bad arguments (-1), a malformed cu_seqlens (-2) or an allocation failure (-3).
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int kda_oracle_version(void);
int kda_oracle_max_threads(void);

/* Whole-sequence recurrence over a packed batch (cu has num_seqs + 1 entries).
 * delta = 1 is KDA; delta = 0 drops the prediction term (gated linear write).
 * S0 may be NULL (zeros); S_out may be NULL.  nthreads <= 0 keeps the OpenMP
 * default. */
int kda_oracle_prefill_f64(int64_t num_seqs, const int64_t *cu, int64_t H,
                           int64_t dk, int64_t dv, double scale, int delta,
                           const double *q, const double *k, const double *v,
                           const double *g, const double *beta,
                           const double *S0, double *o, double *S_out,
                           int nthreads);

/* One token per (n, h): S [N,H,dk,dv] is updated in place, o [N,H,dv]. */
int kda_oracle_decode_step_f64(int64_t N, int64_t H, int64_t dk, int64_t dv,
                               double scale, const double *q, const double *k,
                               const double *v, const double *g,
                               const double *beta, double *S, double *o,
                               int nthreads);

/* Gradients of the prefill above (delta = 1) for a loss with output
 * gradient dO [T_total,H,dv] and final-state gradient dS_T [N,H,dk,dv]
 * (NULL = zeros): dq, dkey, dg [T_total,H,dk], dval [T_total,H,dv],
 * dbeta [T_total,H], dS0 [N,H,dk,dv] (may be NULL).  S0 may be NULL (zeros).
 * seg_len <= 0 selects 64: the forward states are kept at every seg_len-th
 * token and each segment is recomputed from its start. */
int kda_oracle_prefill_backward_f64(int64_t num_seqs, const int64_t *cu, int64_t H,
                                    int64_t dk, int64_t dv, double scale,
                                    const double *q, const double *k, const double *v,
                                    const double *g, const double *beta,
                                    const double *S0, const double *dO,
                                    const double *dS_T, double *dq, double *dkey,
                                    double *dval, double *dg, double *dbeta,
                                    double *dS0, int64_t seg_len, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
