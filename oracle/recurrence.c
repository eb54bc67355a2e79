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
 * The order of steps 1-4 is the one the Muir abstract ("Full text" on the Astral Feed
 * page "Muir: Linear Attention with Sensitivity-Allocated Gating and Matched-Filter
 * Readout") gives for gated delta-rule models: shrink each row of the state by its own
 * decay, remove the decayed state's prediction for the new key, then add the new value,
 * with erase and write under separate gates. The readout
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

/*
 * Reverse mode of the same recurrence (fp64), for the loss
 *   L = sum_t o_t . do_t + <S_T, dS>,
 * written out token by token from the adjoint lambda = dL/dS of the state after each token.
 * For token t (S- = Diag(a_t) S_{t-1}, p, u = w*v - e*p and S_t as in the forward), with
 * q_hat = r * g_t * q_t:
 *   mu      = lambda + q_hat do_t^T         the read of token t adds its cotangent
 *   du      = mu^T k_t                       gradient of u_t
 *   dp      = -e_t * du                      through the erase
 *   dv_t    = w_t * du,  dw_t = v_t * du,  de_t = -p * du
 *   dk_t    = mu u_t + S- dp                 the write and the prediction both use k_t
 *   dq_hat  = S_t do_t
 *   dS-     = mu + k_t dp^T
 *   da_t    = rowsum(S_{t-1} * dS-),   lambda <- Diag(a_t) dS-
 * and dq = r g dq_hat, dg = r q dq_hat, dr = sum over b, t of g q dq_hat; ds0 = the final
 * lambda. la = a * da is returned too (finite where a = 0).
 *
 * Memory stays bounded on long sequences: the forward keeps the state only every SEG tokens
 * and the reverse sweep recomputes each segment's states from its checkpoint (the same
 * operations in the same order, so the same values).
 *
 * Layouts as for the forward; dS may be NULL (zero), s0 may be NULL (zero). Outputs:
 * dq, dk, da, dla, dg [B,T,H,dk]; dv, de, dw [B,T,H,dv]; dr [H,dk]; ds0 [B,H,dk,dv] (may be
 * NULL: not written).
 * Work is split over (b, h) with OpenMP; dr is summed over b afterwards in a fixed order.
 */
#define SEG 128
int oracle_grads_f64(int B, int T, int H, int dk, int dv,
                     const double *q, const double *k, const double *v, const double *a,
                     const double *g, const double *e, const double *w, const double *r,
                     const double *s0, const double *dO, const double *dS,
                     double *dq, double *dk_, double *dv_, double *da, double *dla, double *dg,
                     double *de, double *dw, double *dr, double *ds0, int nthreads)
{
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return 1;
    const size_t dd = (size_t)dk * dv;
    const int nseg = (T + SEG - 1) / SEG;
    double *drp = (double *)calloc((size_t)B * H * dk + 1, sizeof(double));
    if (!drp) return 2;
    int failed = 0;
    if (nthreads <= 0) nthreads = 1;
    _Pragma("omp parallel for schedule(dynamic, 1) num_threads(nthreads)")
    for (long bh = 0; bh < (long)B * H; ++bh) {
        const int b = (int)(bh / H), h = (int)(bh % H);
        double *ck = (double *)malloc(sizeof(double) * dd * (size_t)(nseg > 0 ? nseg : 1));
        double *prev = (double *)malloc(sizeof(double) * dd * SEG);  /* S_{t-1} of the segment */
        double *ps = (double *)malloc(sizeof(double) * (size_t)dv * SEG);
        double *us = (double *)malloc(sizeof(double) * (size_t)dv * SEG);
        double *S = (double *)malloc(sizeof(double) * dd);
        double *lam = (double *)malloc(sizeof(double) * dd);
        double *mu = (double *)malloc(sizeof(double) * dd);
        double *vec = (double *)malloc(sizeof(double) * (size_t)(4 * dk + 4 * dv));
        if (!ck || !prev || !ps || !us || !S || !lam || !mu || !vec) {
            free(ck); free(prev); free(ps); free(us); free(S); free(lam); free(mu); free(vec);
            failed = 1;
            continue;
        }
        double *qh = vec, *dqh = vec + dk, *p = vec + 2 * dk, *u = p + dv, *du = u + dv, *dp = du + dv;
        const double *rh = r + (size_t)h * dk;
        for (size_t x = 0; x < dd; ++x) S[x] = s0 ? s0[((size_t)b * H + h) * dd + x] : 0.0;
        /* one token of the forward: S <- S_t; p and u of the token returned */
        #define FWD_TOKEN(t_, P, U)                                                       \
        do {                                                                              \
            const size_t rk_ = (((size_t)b * T + (t_)) * H + h) * dk;                     \
            const size_t rv_ = (((size_t)b * T + (t_)) * H + h) * dv;                     \
            for (int i = 0; i < dk; ++i)                                                  \
                for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a[rk_ + i];         \
            for (int j = 0; j < dv; ++j) (P)[j] = 0.0;                                    \
            for (int i = 0; i < dk; ++i)                                                  \
                for (int j = 0; j < dv; ++j) (P)[j] += S[(size_t)i * dv + j] * k[rk_ + i]; \
            for (int j = 0; j < dv; ++j) (U)[j] = w[rv_ + j] * v[rv_ + j] - e[rv_ + j] * (P)[j]; \
            for (int i = 0; i < dk; ++i)                                                  \
                for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += k[rk_ + i] * (U)[j]; \
        } while (0)
        for (int t = 0; t < T; ++t) {
            if (t % SEG == 0) memcpy(ck + (size_t)(t / SEG) * dd, S, sizeof(double) * dd);
            FWD_TOKEN(t, p, u);
        }
        for (size_t x = 0; x < dd; ++x) lam[x] = dS ? dS[((size_t)b * H + h) * dd + x] : 0.0;
        for (int sg = nseg - 1; sg >= 0; --sg) {
            const int t0 = sg * SEG, t1 = (t0 + SEG < T) ? t0 + SEG : T;
            memcpy(S, ck + (size_t)sg * dd, sizeof(double) * dd);
            for (int t = t0; t < t1; ++t) {
                memcpy(prev + (size_t)(t - t0) * dd, S, sizeof(double) * dd);
                FWD_TOKEN(t, ps + (size_t)(t - t0) * dv, us + (size_t)(t - t0) * dv);
            }
            for (int t = t1 - 1; t >= t0; --t) {
                const size_t rk = (((size_t)b * T + t) * H + h) * dk;
                const size_t rv = (((size_t)b * T + t) * H + h) * dv;
                const double *Sp = prev + (size_t)(t - t0) * dd;
                const double *pt = ps + (size_t)(t - t0) * dv, *ut = us + (size_t)(t - t0) * dv;
                for (int i = 0; i < dk; ++i) qh[i] = rh[i] * g[rk + i] * q[rk + i];
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        mu[(size_t)i * dv + j] = lam[(size_t)i * dv + j] + qh[i] * dO[rv + j];
                for (int j = 0; j < dv; ++j) du[j] = 0.0;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) du[j] += mu[(size_t)i * dv + j] * k[rk + i];
                for (int j = 0; j < dv; ++j) {
                    dp[j] = -e[rv + j] * du[j];
                    dv_[rv + j] = w[rv + j] * du[j];
                    dw[rv + j] = v[rv + j] * du[j];
                    de[rv + j] = -pt[j] * du[j];
                }
                for (int i = 0; i < dk; ++i) {
                    double acc_k = 0.0, acc_q = 0.0, acc_a = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        const double sm = a[rk + i] * Sp[(size_t)i * dv + j];  /* S- */
                        const double st = sm + k[rk + i] * ut[j];              /* S_t */
                        acc_k += mu[(size_t)i * dv + j] * ut[j] + sm * dp[j];
                        acc_q += st * dO[rv + j];
                        const double dsm = mu[(size_t)i * dv + j] + k[rk + i] * dp[j];
                        acc_a += Sp[(size_t)i * dv + j] * dsm;
                        lam[(size_t)i * dv + j] = a[rk + i] * dsm;
                    }
                    dk_[rk + i] = acc_k;
                    dqh[i] = acc_q;
                    da[rk + i] = acc_a;
                    dla[rk + i] = a[rk + i] * acc_a;
                }
                for (int i = 0; i < dk; ++i) {
                    dq[rk + i] = rh[i] * g[rk + i] * dqh[i];
                    dg[rk + i] = rh[i] * q[rk + i] * dqh[i];
                    drp[((size_t)b * H + h) * dk + i] += g[rk + i] * q[rk + i] * dqh[i];
                }
            }
        }
        #undef FWD_TOKEN
        if (ds0) memcpy(ds0 + ((size_t)b * H + h) * dd, lam, sizeof(double) * dd);
        free(ck); free(prev); free(ps); free(us); free(S); free(lam); free(mu); free(vec);
    }
    for (int h = 0; h < H; ++h)
        for (int i = 0; i < dk; ++i) {
            double s = 0.0;
            for (int b = 0; b < B; ++b) s += drp[((size_t)b * H + h) * dk + i];
            dr[(size_t)h * dk + i] = s;
        }
    free(drp);
    return failed ? 2 : 0;
}
#undef SEG
