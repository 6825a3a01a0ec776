/*
 * CPU oracle for the gated delta rule of Kimi Delta Attention (KDA) — TEST
 * INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg may load this file's library; the product path never does.
 *
 * What it computes (the plain definition, written out token by token in fp64):
 *
 *   "Kimi Delta Attention" SM100 prefill digest (sglang PR 27488), sections
 *   "功能与动机" (motivation: per-channel decay gate, outputs checked against a
 *   token-by-token baseline) and "风险与影响" (risks: o error measured against
 *   that token-by-token baseline).  The pages never print the recurrence; the
 *   one used here is the per-head state update of KDA:
 *
 *       S'_t = Diag(exp g_t) S_{t-1}                    (decay first)
 *       u_t  = beta_t (v_t - S'_t^T k_t)                (delta-rule residual)
 *       S_t  = S'_t + k_t u_t^T                         (rank-1 write)
 *       o_t  = scale * S_t^T q_t                        (read out after the write)
 *
 *   S is K x V per (sequence, value head).  GDN's scalar gate is the special
 *   case where g_t is one number per (token, head) applied to every channel
 *   ("GDN" pool-mode digest, sglang PR 30169, key-code test: gate shape
 *   [1, T, Hv]).
 *
 * Storage conventions (pool-mode digest, key-code test: initial state
 * [N, Hv, V, K]): states are stored V-major with K contiguous, i.e. the
 * transpose of the math S.  q, k are [T, Hk, K]; v is [T, Hv, V]; g is
 * [T, Hv, K] (per channel) or [T, Hv] (scalar); beta is [T, Hv].  Value head h
 * reads key head h / (Hv / Hk).  Sequences are packed by cu_seqlens [N + 1].
 *
 * q, k, v and the initial states are float (bf16 and fp32 convert to float
 * exactly); g and beta are double, so that gates computed in fp64 from their
 * raw inputs (oracle.gate_activation) enter unrounded.  Every operation is
 * done in double.  No blocking, no chunking, no reordering: one token at a
 * time, in order.
 *
 * parity pinned by tests/test_oracle_pins.py (closed forms, invariants,
 * brute-force transition-matrix form, chunked-vs-recurrent equivalence).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One (sequence, value head) unit: run the recurrence over tokens [t0, t1). */
static void run_unit(int32_t t0, int32_t t1, int32_t h, int32_t hk_idx,
                     int32_t hk, int32_t hv, int32_t dk, int32_t dv,
                     int gate_scalar, double scale,
                     const float *q, const float *k, const float *v,
                     const double *g, const double *beta,
                     const float *h0_unit, /* [dv, dk] or NULL */
                     double *o, double *ht_unit, /* [dv, dk] or NULL */
                     double *S, double *pred, double *u)
{
    /* S is the math state, K x V, row c holds channel c: S[c * dv + j]. */
    for (int32_t c = 0; c < dk; ++c)
        for (int32_t j = 0; j < dv; ++j)
            S[(size_t)c * dv + j] = h0_unit ? (double)h0_unit[(size_t)j * dk + c] : 0.0;

    for (int32_t t = t0; t < t1; ++t) {
        const float *qt = q + ((size_t)t * hk + hk_idx) * dk;
        const float *kt = k + ((size_t)t * hk + hk_idx) * dk;
        const float *vt = v + ((size_t)t * hv + h) * dv;
        const double bt = beta[(size_t)t * hv + h];

        /* decay: row c of S scales by exp(g_t[c]) */
        for (int32_t c = 0; c < dk; ++c) {
            const double gc = gate_scalar ? g[(size_t)t * hv + h]
                                          : g[((size_t)t * hv + h) * dk + c];
            const double a = exp(gc);
            double *row = S + (size_t)c * dv;
            for (int32_t j = 0; j < dv; ++j) row[j] *= a;
        }
        /* prediction S'^T k */
        for (int32_t j = 0; j < dv; ++j) pred[j] = 0.0;
        for (int32_t c = 0; c < dk; ++c) {
            const double kc = (double)kt[c];
            const double *row = S + (size_t)c * dv;
            for (int32_t j = 0; j < dv; ++j) pred[j] += row[j] * kc;
        }
        /* residual and rank-1 write */
        for (int32_t j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - pred[j]);
        for (int32_t c = 0; c < dk; ++c) {
            const double kc = (double)kt[c];
            double *row = S + (size_t)c * dv;
            for (int32_t j = 0; j < dv; ++j) row[j] += kc * u[j];
        }
        /* read out after the write */
        double *ot = o + ((size_t)t * hv + h) * dv;
        for (int32_t j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int32_t c = 0; c < dk; ++c) {
            const double qc = (double)qt[c];
            const double *row = S + (size_t)c * dv;
            for (int32_t j = 0; j < dv; ++j) ot[j] += row[j] * qc;
        }
        for (int32_t j = 0; j < dv; ++j) ot[j] *= scale;
    }

    if (ht_unit)
        for (int32_t j = 0; j < dv; ++j)
            for (int32_t c = 0; c < dk; ++c)
                ht_unit[(size_t)j * dk + c] = S[(size_t)c * dv + j];
}

/*
 * Packed variable-length prefill.
 *   cu_seqlens : [num_seqs + 1] host int32, cu[0] = 0, non-decreasing
 *   h0         : [num_seqs, hv, dv, dk] float, or NULL for zero initial states
 *   o          : [T, hv, dv] double (T = cu[num_seqs])
 *   ht         : [num_seqs, hv, dv, dk] double, or NULL
 *   nthreads   : OpenMP threads (<= 0: library default)
 * Returns 0, or -1 on a shape error (hv % hk != 0, non-positive dims).
 */
int kdaref_prefill(int32_t num_seqs, const int32_t *cu_seqlens,
                   int32_t hk, int32_t hv, int32_t dk, int32_t dv,
                   int32_t gate_scalar, double scale,
                   const float *q, const float *k, const float *v,
                   const double *g, const double *beta, const float *h0,
                   double *o, double *ht, int32_t nthreads)
{
    if (num_seqs < 0 || hk <= 0 || hv <= 0 || dk <= 0 || dv <= 0 || hv % hk != 0)
        return -1;
    const int32_t group = hv / hk;
    const long units = (long)num_seqs * hv;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *pred = (double *)malloc(sizeof(double) * (size_t)dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(dynamic, 1)
        for (long unit = 0; unit < units; ++unit) {
            const int32_t n = (int32_t)(unit / hv), h = (int32_t)(unit % hv);
            const size_t st = ((size_t)n * hv + h) * (size_t)dv * dk;
            run_unit(cu_seqlens[n], cu_seqlens[n + 1], h, h / group, hk, hv, dk, dv,
                     gate_scalar, scale, q, k, v, g, beta,
                     h0 ? h0 + st : NULL, o, ht ? ht + st : NULL, S, pred, u);
        }
        free(S);
        free(pred);
        free(u);
    }
    return 0;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int kdaref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
