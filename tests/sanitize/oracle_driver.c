/* Runs the CPU oracle's C code (token recurrence in fp64 and fp32, and its adjoint) on small
 * seeded inputs, for a build with the address and undefined-behaviour sanitizers: several
 * thread counts, with and without an initial state and a final-state gradient, T spanning
 * several checkpoint segments, and the invalid-size return codes. Exit status 0 when every
 * call succeeds and every output is finite. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_recurrent_f64(int B, int T, int H, int dk, int dv, const double *q, const double *k,
                         const double *v, const double *a, const double *g, const double *e,
                         const double *w, const double *r, const double *s0, double *o,
                         double *s_out, int nthreads);
int oracle_recurrent_f32(int B, int T, int H, int dk, int dv, const float *q, const float *k,
                         const float *v, const float *a, const float *g, const float *e,
                         const float *w, const float *r, const float *s0, float *o,
                         float *s_out, int nthreads);
int oracle_grads_f64(int B, int T, int H, int dk, int dv, const double *q, const double *k,
                     const double *v, const double *a, const double *g, const double *e,
                     const double *w, const double *r, const double *s0, const double *dO,
                     const double *dS, double *dq, double *dk_, double *dv_, double *da,
                     double *dla, double *dg, double *de, double *dw, double *dr, double *ds0,
                     int nthreads);

static unsigned long long rng = 88172645463325252ull;
static double uni(void) { /* xorshift64 */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}
static double *fill(size_t n, double lo, double hi) {
    double *p = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * uni();
    return p;
}
static int finite(const double *p, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static int run(int B, int T, int H, int d, int with_state, int nthreads) {
    const size_t nt = (size_t)B * T * H * d, ns = (size_t)B * H * d * d, nr = (size_t)H * d;
    double *q = fill(nt, -1, 1), *k = fill(nt, -0.3, 0.3), *v = fill(nt, -1, 1);
    double *a = fill(nt, 0.5, 1), *g = fill(nt, 0, 1), *e = fill(nt, 0, 1), *w = fill(nt, 0, 1);
    double *r = fill(nr, 0.5, 1.5), *s0 = with_state ? fill(ns, -0.5, 0.5) : NULL;
    double *dO = fill(nt, -1, 1), *dS = with_state ? fill(ns, -1, 1) : NULL;
    double *o = malloc(nt * sizeof(double)), *s = malloc(ns * sizeof(double));
    double *gr[8];
    for (int i = 0; i < 8; ++i) gr[i] = malloc(nt * sizeof(double));
    double *dr = malloc(nr * sizeof(double)), *ds0 = malloc(ns * sizeof(double));
    float *qf = malloc(nt * sizeof(float)), *of = malloc(nt * sizeof(float));
    float *ff[7], *rf = malloc(nr * sizeof(float)), *sf = malloc(ns * sizeof(float));
    const double *src[7] = {k, v, a, g, e, w, q};
    for (int i = 0; i < 7; ++i) {
        ff[i] = malloc(nt * sizeof(float));
        for (size_t j = 0; j < nt; ++j) ff[i][j] = (float)src[i][j];
    }
    for (size_t j = 0; j < nt; ++j) qf[j] = (float)q[j];
    for (size_t j = 0; j < nr; ++j) rf[j] = (float)r[j];
    int bad = 0;
    bad |= oracle_recurrent_f64(B, T, H, d, d, q, k, v, a, g, e, w, r, s0, o, s, nthreads) != 0;
    bad |= !finite(o, nt) || !finite(s, ns);
    bad |= oracle_recurrent_f32(B, T, H, d, d, qf, ff[0], ff[1], ff[2], ff[3], ff[4], ff[5], rf,
                                NULL, of, sf, nthreads) != 0;
    bad |= oracle_grads_f64(B, T, H, d, d, q, k, v, a, g, e, w, r, s0, dO, dS, gr[0], gr[1], gr[2],
                            gr[3], gr[4], gr[5], gr[6], gr[7], dr, with_state ? ds0 : NULL,
                            nthreads) != 0;
    for (int i = 0; i < 8; ++i) bad |= !finite(gr[i], nt);
    bad |= !finite(dr, nr);
    if (bad) printf("FAIL B=%d T=%d H=%d d=%d state=%d threads=%d\n", B, T, H, d, with_state, nthreads);
    double *all[] = {q, k, v, a, g, e, w, r, s0, dO, dS, o, s, dr, ds0};
    for (size_t i = 0; i < sizeof all / sizeof all[0]; ++i) free(all[i]);
    for (int i = 0; i < 8; ++i) free(gr[i]);
    for (int i = 0; i < 7; ++i) free(ff[i]);
    free(qf); free(of); free(rf); free(sf);
    return bad;
}

int main(void) {
    int bad = 0;
    bad |= run(1, 1, 1, 4, 0, 1);
    bad |= run(2, 37, 3, 8, 1, 1);
    bad |= run(2, 37, 3, 8, 1, 3);
    bad |= run(1, 300, 2, 20, 1, 4); /* several checkpoint segments, a partial column block */
    bad |= run(1, 0, 2, 8, 1, 2);
    /* Invalid sizes are refused, not read. */
    bad |= oracle_recurrent_f64(-1, 4, 1, 4, 4, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                NULL, NULL, NULL, 1) == 0;
    bad |= oracle_recurrent_f64(1, 4, 0, 4, 4, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                NULL, NULL, NULL, 1) == 0;
    printf("%s\n", bad ? "oracle driver: failures" : "oracle driver: ok");
    return bad;
}
