/*
 * CPU oracle: the plain token-by-token gated delta rule with matched-filter readout.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link or call
 * this file; it shares no code with the HIP library.
 *
 * What it computes (per batch b, head h; state S is dk x dv, rows = key channels):
 *   for t = 1..T:
 *     1. S <- Diag(a_t) S                      decay every row by its own factor
 *     2. p <- S^T k_t                          the decayed state's prediction for k_t
 *     3. S <- S - k_t (e_t * p)^T              erase that prediction, per value channel
 *     4. S <- S + k_t (w_t * v_t)^T            write the gated value
 *     5. o_t <- S^T (r * g_t * q_t)            matched-filter read of the updated state
 * The order decay -> erase the prediction for the incoming key -> write comes from
 * the Muir abstract ("Full text" on the Astral Feed page "Muir: Linear Attention with
 * Sensitivity-Allocated Gating and Matched-Filter Readout"): gated delta-rule models
 * decay the state and erase its prediction for an incoming key before writing a new
 * value, with channel-wise decay and decoupled erase and write gates. The readout
 * (a static per-row scale r from each row's expected energy times a per-token query
 * gate g) is from the openai-hub news page, section on matched-filter readout, and the
 * liuch.name summary, first bullet. The erase and write gates act on value channels,
 * the decay and query gate on key channels; the read is inclusive of token t.
 *
 * Layouts (all contiguous, row-major):
 *   q, k, a, g : [B, T, H, dk]      v, e, w : [B, T, H, dv]      r : [H, dk]
 *   s0, s_out  : [B, H, dk, dv]     o       : [B, T, H, dv]
 * s0 may be NULL (zero initial state). Work is split over independent
 * (b, h, value-column block) chains with OpenMP; each chain runs the token loop.
 */
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define COL_BLOCK 16

#define DEFINE_RECURRENT(NAME, REAL)                                                    \
int NAME(int B, int T, int H, int dk, int dv,                                           \
         const REAL *q, const REAL *k, const REAL *v,                                   \
         const REAL *a, const REAL *g, const REAL *e, const REAL *w,                    \
         const REAL *r, const REAL *s0, REAL *o, REAL *s_out, int nthreads)             \
{                                                                                       \
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return 1;                      \
    const int nblk = (dv + COL_BLOCK - 1) / COL_BLOCK;                                  \
    const long nchains = (long)B * H * nblk;                                            \
    int failed = 0;                                                                     \
    if (nthreads <= 0) nthreads = 1;                                                    \
    _Pragma("omp parallel for schedule(dynamic, 1) num_threads(nthreads)")              \
    for (long c = 0; c < nchains; ++c) {                                                \
        const int blk = (int)(c % nblk);                                                \
        const int h = (int)((c / nblk) % H);                                            \
        const int b = (int)(c / ((long)nblk * H));                                      \
        const int j0 = blk * COL_BLOCK;                                                 \
        const int nj = (dv - j0) < COL_BLOCK ? (dv - j0) : COL_BLOCK;                   \
        REAL *S = (REAL *)malloc(sizeof(REAL) * (size_t)dk * COL_BLOCK);                \
        REAL *qh = (REAL *)malloc(sizeof(REAL) * (size_t)dk);                           \
        if (!S || !qh) { free(S); free(qh); failed = 1; continue; }                     \
        for (int i = 0; i < dk; ++i)                                                    \
            for (int j = 0; j < nj; ++j)                                                \
                S[i * COL_BLOCK + j] = s0 ?                                             \
                    s0[(((size_t)b * H + h) * dk + i) * dv + j0 + j] : (REAL)0;         \
        for (int t = 0; t < T; ++t) {                                                   \
            const size_t rk = (((size_t)b * T + t) * H + h) * dk;                       \
            const size_t rv = (((size_t)b * T + t) * H + h) * dv;                       \
            REAL p[COL_BLOCK];                                                          \
            /* 1. decay */                                                              \
            for (int i = 0; i < dk; ++i)                                                \
                for (int j = 0; j < nj; ++j) S[i * COL_BLOCK + j] *= a[rk + i];         \
            /* 2. prediction for k_t from the decayed state */                          \
            for (int j = 0; j < nj; ++j) p[j] = 0;                                      \
            for (int i = 0; i < dk; ++i)                                                \
                for (int j = 0; j < nj; ++j) p[j] += S[i * COL_BLOCK + j] * k[rk + i];  \
            /* 3. erase e_t * p along k_t */                                            \
            for (int i = 0; i < dk; ++i)                                                \
                for (int j = 0; j < nj; ++j)                                            \
                    S[i * COL_BLOCK + j] -= k[rk + i] * (e[rv + j0 + j] * p[j]);        \
            /* 4. write w_t * v_t along k_t */                                          \
            for (int i = 0; i < dk; ++i)                                                \
                for (int j = 0; j < nj; ++j)                                            \
                    S[i * COL_BLOCK + j] += k[rk + i] * (w[rv + j0 + j] * v[rv + j0 + j]); \
            /* 5. matched-filter read: o_t = S^T (r * g_t * q_t) */                     \
            for (int i = 0; i < dk; ++i)                                                \
                qh[i] = r[(size_t)h * dk + i] * g[rk + i] * q[rk + i];                  \
            for (int j = 0; j < nj; ++j) {                                              \
                REAL acc = 0;                                                           \
                for (int i = 0; i < dk; ++i) acc += S[i * COL_BLOCK + j] * qh[i];       \
                o[rv + j0 + j] = acc;                                                   \
            }                                                                           \
        }                                                                               \
        if (s_out)                                                                      \
            for (int i = 0; i < dk; ++i)                                                \
                for (int j = 0; j < nj; ++j)                                            \
                    s_out[(((size_t)b * H + h) * dk + i) * dv + j0 + j] =               \
                        S[i * COL_BLOCK + j];                                           \
        free(S);                                                                        \
        free(qh);                                                                       \
    }                                                                                   \
    return failed ? 2 : 0;                                                              \
}

DEFINE_RECURRENT(oracle_recurrent_f64, double)
DEFINE_RECURRENT(oracle_recurrent_f32, float)

/* Number of threads OpenMP would use by default (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
