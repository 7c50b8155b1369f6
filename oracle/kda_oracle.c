/*
 * kda_oracle.c -- fp64 CPU oracle for the Kimi Delta Attention (KDA) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or constant with the HIP implementation.
 *
 * What it computes (one sequence, one head, token by token, all in double):
 *   Source: course page "线性注意力与 KDA" (ai.air7.fun, Day 19), section 3,
 *   the two displayed update equations, and section 2 for the read-out:
 *     decay      S~  = Diag(alpha_t) S_{t-1}      alpha_t = exp(g_t), one factor per key channel
 *     delta      S_t = S~ + beta_t * k_t (v_t - S~^T k_t)^T
 *     read-out   o_t = scale * S_t^T q_t          (the updated state is read)
 *   The per-channel decay acts on the key axis (page "Kimi K3 注意力三件套",
 *   KDA section: alpha_t in [0,1]^{d_k}; blog post ciyuanerhao post-114,
 *   chapter 4: the per-channel factor scales the rows of a d_k x d_v state).
 *   State orientation is K-major: S[i*dv + j] couples key channel i with value
 *   channel j (the chapter 3 DeltaNet of that blog keeps its memory d_k x d_v).
 *
 * Inputs are the stored fp32 (or bf16-valued fp32) numbers, converted to double
 * exactly.  Nothing is clamped: NaN and Inf propagate.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

/*
 * One chain of L tokens.
 *   q, k, g : token t, key channel i at  x[t*ld + i]      (i < dk)
 *   v       : token t, value channel j at v[t*ldv + j]     (j < dv)
 *   beta    : token t at beta[t*ldb]
 *   S0      : [dk*dv] initial state, or NULL for zero
 *   o       : token t, value channel j at o[t*ldo + j]    (double)
 *   S_out   : [dk*dv] final state (double); may be NULL
 * Returns 0 on success, -1 if the work buffers could not be allocated.
 */
int kda_oracle_chain(long L, int dk, int dv,
                     const float *q, long ldq,
                     const float *k, long ldk,
                     const float *v, long ldv,
                     const float *g, long ldg,
                     const float *beta, long ldb,
                     double scale,
                     const float *S0,
                     double *o, long ldo,
                     double *S_out)
{
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
    double *kt = (double *)malloc(sizeof(double) * (size_t)dk);
    double *qt = (double *)malloc(sizeof(double) * (size_t)dk);
    double *u = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!S || !kt || !qt || !u) {
        free(S); free(kt); free(qt); free(u);
        return -1;
    }
    for (long e = 0; e < (long)dk * dv; ++e)
        S[e] = S0 ? (double)S0[e] : 0.0;

    for (long t = 0; t < L; ++t) {
        const float *qr = q + t * ldq, *kr = k + t * ldk, *vr = v + t * ldv, *gr = g + t * ldg;
        const double b = (double)beta[t * ldb];
        for (int i = 0; i < dk; ++i) {
            kt[i] = (double)kr[i];
            qt[i] = (double)qr[i];
        }
        /* decay: row i of S (key channel i) is multiplied by alpha_i = exp(g_i) */
        for (int i = 0; i < dk; ++i) {
            const double a = exp((double)gr[i]);
            double *row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j)
                row[j] *= a;
        }
        /* prediction of the decayed memory for key k_t: p = S~^T k_t, then u = beta (v - p) */
        for (int j = 0; j < dv; ++j)
            u[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double *row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j)
                u[j] += row[j] * kt[i];
        }
        for (int j = 0; j < dv; ++j)
            u[j] = b * ((double)vr[j] - u[j]);
        /* write the correction: S = S~ + k_t u^T */
        for (int i = 0; i < dk; ++i) {
            double *row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j)
                row[j] += kt[i] * u[j];
        }
        /* read-out with the updated state: o_t = scale * S_t^T q_t */
        double *orow = o + t * ldo;
        for (int j = 0; j < dv; ++j)
            orow[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double *row = S + (size_t)i * dv;
            for (int j = 0; j < dv; ++j)
                orow[j] += row[j] * qt[i];
        }
        for (int j = 0; j < dv; ++j)
            orow[j] *= scale;
    }
    if (S_out)
        memcpy(S_out, S, sizeof(double) * (size_t)dk * (size_t)dv);
    free(S); free(kt); free(qt); free(u);
    return 0;
}
