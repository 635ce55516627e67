/*
 * Float64 CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the HIP path, and the HIP path never calls it.
 *
 * What it computes: the per-token recurrence of "Linear attention"
 * (arsalanzafar.ai), section "How it works", Eqs. (1)-(4), in the
 * d_k x d_v state convention of that page (state stored as keys x values):
 *
 *   (1) S'    = alpha_t * S_{t-1}                      decay
 *   (2) vhat  = S'^T k_t                               predict from the decayed state
 *   (3) S_t   = S' + beta_t * k_t (v_t - vhat)^T       correct along the key
 *   (4) o_t   = S_t^T q_t                              read after the write
 *
 * The same update appears as "decay, predict, correct, read" in "How linear
 * attention works: a small memory matrix and the gated delta rule", section
 * "The gated delta rule" (there with values x keys; transposed here), and as
 * the decayed delta update of "From KV Cache to a State Matrix: Linear
 * Attention and DeltaNet", section "Why DeltaNet may forget too slowly".
 *
 * With delta == 0 step (2) is skipped (vhat := 0): the additive rule
 * S_t = alpha_t S_{t-1} + beta_t k_t v_t^T.  That mode exists only so that
 * tests can pin the oracle against unnormalised causal linear attention
 * ("From KV Cache to a State Matrix", section "From attention weights to a
 * state matrix").
 *
 * Layout: unit-major and contiguous.  A unit is one (sequence, value head).
 *   q, k   [n_units][T][d_k]      v, o   [n_units][T][d_v]
 *   alpha, beta [n_units][T]      h0, hT [n_units][d_k][d_v]  (row-major, d_v fastest)
 * h0 may be NULL (S_0 = 0).  hT may be NULL.
 *
 * Mutants: building with -DORACLE_MUTANT=<n> plants one deliberate mistake so
 * that a test can show the pins catch it.  The default build has none.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

static void gdn_one_unit(int64_t T, int64_t dk, int64_t dv,
                         const double *q, const double *k, const double *v,
                         const double *alpha, const double *beta,
                         const double *h0, int delta,
                         double *o, double *hT, double *S, double *vhat) {
    int64_t i, j, t;
    if (h0)
        memcpy(S, h0, sizeof(double) * (size_t)(dk * dv));
    else
        memset(S, 0, sizeof(double) * (size_t)(dk * dv));

    for (t = 0; t < T; ++t) {
        const double *qt = q + t * dk;
        const double *kt = k + t * dk;
        const double *vt = v + t * dv;
        double *ot = o + t * dv;
        const double a = alpha[t];
        const double b = beta[t];

#if ORACLE_MUTANT == 1
        /* mutant: predict from the undecayed state S_{t-1} */
        for (j = 0; j < dv; ++j) {
            vhat[j] = 0.0;
            if (delta)
                for (i = 0; i < dk; ++i) vhat[j] += S[i * dv + j] * kt[i];
        }
#endif
        /* Eq. (1): decay the whole state. */
        for (i = 0; i < dk * dv; ++i) S[i] *= a;

        /* Eq. (2): what the decayed memory returns for the key. */
#if ORACLE_MUTANT != 1
        for (j = 0; j < dv; ++j) vhat[j] = 0.0;
        if (delta)
            for (i = 0; i < dk; ++i)
                for (j = 0; j < dv; ++j) vhat[j] += S[i * dv + j] * kt[i];
#endif

#if ORACLE_MUTANT == 2
        /* mutant: read with the query before the write */
        for (j = 0; j < dv; ++j) {
            ot[j] = 0.0;
            for (i = 0; i < dk; ++i) ot[j] += S[i * dv + j] * qt[i];
        }
#endif
        /* Eq. (3): write the correction along the key. */
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j) {
#if ORACLE_MUTANT == 3
                /* mutant: the correction's sign flipped */
                S[i * dv + j] += b * kt[i] * (vhat[j] - vt[j]);
#elif ORACLE_MUTANT == 4
                /* mutant: the write is decayed too */
                S[i * dv + j] += a * b * kt[i] * (vt[j] - vhat[j]);
#elif ORACLE_MUTANT == 5
                /* mutant: the write uses the query instead of the key */
                S[i * dv + j] += b * qt[i] * (vt[j] - vhat[j]);
#else
                S[i * dv + j] += b * kt[i] * (vt[j] - vhat[j]);
#endif
            }

        /* Eq. (4): read the updated state with the query. */
#if ORACLE_MUTANT != 2
        for (j = 0; j < dv; ++j) ot[j] = 0.0;
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j) ot[j] += S[i * dv + j] * qt[i];
#endif
    }
    if (hT) memcpy(hT, S, sizeof(double) * (size_t)(dk * dv));
}

/* Runs every unit independently ("each such head and sequence has its own
 * state", "How linear attention works", section "What every dimension
 * means").  Returns 0 on success, -1 on bad arguments or allocation failure. */
int gdn_oracle_forward(int64_t n_units, int64_t T, int64_t dk, int64_t dv,
                       const double *q, const double *k, const double *v,
                       const double *alpha, const double *beta,
                       const double *h0, int delta,
                       double *o, double *hT, int n_threads) {
    int64_t u;
    int failed = 0;
    if (n_units < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    if (n_units == 0) return 0;
    if (!q || !k || !v || !alpha || !beta || !o) return -1;
    if (n_threads < 1) n_threads = 1;

#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(| : failed)
    for (u = 0; u < n_units; ++u) {
        double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
        double *vhat = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !vhat) {
            failed |= 1;
        } else {
            gdn_one_unit(T, dk, dv, q + u * T * dk, k + u * T * dk, v + u * T * dv,
                         alpha + u * T, beta + u * T, h0 ? h0 + u * dk * dv : NULL, delta,
                         o + u * T * dv, hT ? hT + u * dk * dv : NULL, S, vhat);
        }
        free(S);
        free(vhat);
    }
    return failed ? -1 : 0;
}

int gdn_oracle_mutant(void) { return ORACLE_MUTANT; }
