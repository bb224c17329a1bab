/* Sanitizer driver for the C oracle (oracle/ssm_oracle.c built with AddressSanitizer and
 * UndefinedBehaviorSanitizer). Calls every exported oracle function on small seeded inputs --
 * odd sizes, one-entry and full windows, empty snapshot lists, two OpenMP threads -- and checks
 * the identities the oracle's own pins rest on (replay and flush forms against stepping, the
 * speculative rounds against stepping the accepted stream), so that an out-of-bounds index or an
 * uninitialised read in any of them is caught here, and a result that changed with it too. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_set_threads(int n);
void orc_m2_sequential_batch(int nh, int P, int N, int T, const double *A, const double *D,
                             const double *h0, const double *x, const double *B, const double *C,
                             const double *dt, double *y, double *h_out, int nsnap,
                             const int *snap_after, double *snaps);
void orc_m2_replay_output(int P, int N, int k, double A, double D, const double *hc,
                          const double *x, const double *B, const double *Ck, const double *dt,
                          double *y);
void orc_m2_flush(int P, int N, int L, double A, const double *hc, const double *x,
                  const double *B, const double *dt, double *out);
void orc_m2_spec_rounds_batch(int nh, int P, int N, int R, int S, const double *A, const double *D,
                              const double *h0, const double *x, const double *B, const double *C,
                              const double *dt, const int *accept, double *y, double *h_out,
                              int nsnap, const int *snap_after, double *snaps);
void orc_gdn_sequential_batch(int nh, int dv, int dk, int T, double scale, const double *S0,
                              const double *q, const double *k, const double *v,
                              const double *beta, const double *g, double *o, double *S_out,
                              int nsnap, const int *snap_after, double *snaps);
void orc_kda_sequential_batch(int nh, int dv, int dk, int T, double scale, const double *S0,
                              const double *q, const double *k, const double *v,
                              const double *beta, const double *g, double *o, double *S_out,
                              int nsnap, const int *snap_after, double *snaps);
void orc_gdn_replay_output(int dv, int dk, int kk, double scale, const double *Sc,
                           const double *qk, const double *k, const double *v, const double *beta,
                           const double *g, double *o);
void orc_kda_replay_output(int dv, int dk, int kk, double scale, const double *Sc,
                           const double *qk, const double *k, const double *v, const double *beta,
                           const double *g, double *o);
void orc_replay_query(int dv, int dk, int kk, int kda, const double *qk, const double *k,
                      const double *v, const double *beta, const double *g, double *r);
void orc_gdn_flush(int dv, int dk, int L, const double *Sc, const double *k, const double *v,
                   const double *beta, const double *g, double *S_new);
void orc_gdn_spec_rounds_batch(int nh, int dv, int dk, int R, int S, double scale,
                               const double *S0, const double *q, const double *k, const double *v,
                               const double *beta, const double *g, const int *accept, double *o,
                               double *S_out, int nsnap, const int *snap_after, double *snaps);
void orc_kda_spec_rounds_batch(int nh, int dv, int dk, int R, int S, double scale,
                               const double *S0, const double *q, const double *k, const double *v,
                               const double *beta, const double *g, const int *accept, double *o,
                               double *S_out, int nsnap, const int *snap_after, double *snaps);

static unsigned long long rng = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [0, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) * (1.0 / 9007199254740992.0);
}
static double *arr(size_t n, double lo, double hi) {
    double *a = (double *)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) a[i] = lo + (hi - lo) * urand();
    return a;
}
static int fails = 0;
static void close_to(const double *a, const double *b, size_t n, double tol, const char *what) {
    double worst = 0;
    for (size_t i = 0; i < n; ++i) {
        const double d = fabs(a[i] - b[i]) / (1.0 + fabs(b[i]));
        if (!(d <= worst)) worst = d;
    }
    if (!(worst <= tol)) { fprintf(stderr, "%s: worst %.3g > %.1g\n", what, worst, tol); ++fails; }
}

static void mamba2(int P, int N, int T, int L) {
    const int nh = 3;
    double *A = arr(nh, -3, -0.2), *D = arr(nh, -1, 1), *h0 = arr((size_t)nh * P * N, -0.3, 0.3);
    double *x = arr((size_t)nh * T * P, -1, 1), *B = arr((size_t)nh * T * N, -0.3, 0.3);
    double *C = arr((size_t)nh * T * N, -0.3, 0.3), *dt = arr((size_t)nh * T, 0.05, 0.5);
    double *y = calloc((size_t)nh * T * P, sizeof(double)), *hT = calloc((size_t)nh * P * N, sizeof(double));
    int snap[1] = {L};
    double *sn = calloc((size_t)nh * P * N, sizeof(double));
    orc_m2_sequential_batch(nh, P, N, T, A, D, h0, x, B, C, dt, y, hT, 1, snap, sn);
    orc_m2_sequential_batch(nh, P, N, T, A, D, NULL, x, B, C, dt, y, hT, 0, NULL, NULL);
    orc_m2_sequential_batch(nh, P, N, T, A, D, h0, x, B, C, dt, y, hT, 1, snap, sn);
    double *yr = calloc(P, sizeof(double)), *hf = calloc((size_t)P * N, sizeof(double));
    for (int i = 0; i < nh; ++i) {
        const double *xi = x + (size_t)i * T * P, *Bi = B + (size_t)i * T * N, *dti = dt + (size_t)i * T;
        for (int k = 1; k <= L; ++k) { /* replay from the initial state equals stepping */
            orc_m2_replay_output(P, N, k, A[i], D[i], h0 + (size_t)i * P * N, xi, Bi,
                                 C + ((size_t)i * T + k - 1) * N, dti, yr);
            close_to(yr, y + ((size_t)i * T + k - 1) * P, P, 1e-12, "mamba2 replay");
        }
        orc_m2_flush(P, N, L, A[i], h0 + (size_t)i * P * N, xi, Bi, dti, hf);
        close_to(hf, sn + (size_t)i * P * N, (size_t)P * N, 1e-12, "mamba2 flush");
    }
    /* speculative rounds: all accepted equals stepping the drafts */
    const int R = 2, S = T / 2;
    int *acc = malloc(sizeof(int) * nh * R);
    for (int i = 0; i < nh * R; ++i) acc[i] = S;
    double *ys = calloc((size_t)nh * R * S * P, sizeof(double)), *hs = calloc((size_t)nh * P * N, sizeof(double));
    orc_m2_spec_rounds_batch(nh, P, N, R, S, A, D, h0, x, B, C, dt, acc, ys, hs, 0, NULL, NULL);
    close_to(hs, hT, (size_t)nh * P * N, 1e-12, "mamba2 spec rounds");
    free(A); free(D); free(h0); free(x); free(B); free(C); free(dt); free(y); free(hT); free(sn);
    free(yr); free(hf); free(acc); free(ys); free(hs);
}

static void delta(int kda, int dv, int dk, int T, int L) {
    const int nh = 2, gd = kda ? dk : 1;
    double *S0 = arr((size_t)nh * dv * dk, -0.3, 0.3), *q = arr((size_t)nh * T * dk, -0.2, 0.2);
    double *k = arr((size_t)nh * T * dk, -0.2, 0.2), *v = arr((size_t)nh * T * dv, -1, 1);
    double *beta = arr((size_t)nh * T, 0.1, 0.9), *g = arr((size_t)nh * T * gd, -1.5, -0.01);
    double *o = calloc((size_t)nh * T * dv, sizeof(double)), *ST = calloc((size_t)nh * dv * dk, sizeof(double));
    int snap[2] = {L, T};
    double *sn = calloc((size_t)2 * nh * dv * dk, sizeof(double));
    if (kda) orc_kda_sequential_batch(nh, dv, dk, T, 0.7, S0, q, k, v, beta, g, o, ST, 2, snap, sn);
    else orc_gdn_sequential_batch(nh, dv, dk, T, 0.7, S0, q, k, v, beta, g, o, ST, 2, snap, sn);
    double *orr = calloc(dv, sizeof(double)), *r = calloc(dk, sizeof(double));
    for (int i = 0; i < nh; ++i) {
        const double *ki = k + (size_t)i * T * dk, *vi = v + (size_t)i * T * dv;
        const double *bi = beta + (size_t)i * T, *gi = g + (size_t)i * T * gd;
        for (int kk = 1; kk <= L; ++kk) {
            const double *qk = q + ((size_t)i * T + kk - 1) * dk;
            if (kda) orc_kda_replay_output(dv, dk, kk, 0.7, S0 + (size_t)i * dv * dk, qk, ki, vi, bi, gi, orr);
            else orc_gdn_replay_output(dv, dk, kk, 0.7, S0 + (size_t)i * dv * dk, qk, ki, vi, bi, gi, orr);
            close_to(orr, o + ((size_t)i * T + kk - 1) * dv, dv, 1e-12, "delta replay");
            orc_replay_query(dv, dk, kk, kda, qk, ki, vi, bi, gi, r);
        }
        if (!kda) {
            double *Sf = calloc((size_t)dv * dk, sizeof(double));
            orc_gdn_flush(dv, dk, L, S0 + (size_t)i * dv * dk, ki, vi, bi, gi, Sf);
            close_to(Sf, sn + ((size_t)i * 2) * dv * dk, (size_t)dv * dk, 1e-12, "gdn flush");
            free(Sf);
        }
    }
    const int R = 2, S = T / 2;
    int *acc = malloc(sizeof(int) * nh * R);
    for (int i = 0; i < nh * R; ++i) acc[i] = S;
    double *os = calloc((size_t)nh * R * S * dv, sizeof(double)), *Ss = calloc((size_t)nh * dv * dk, sizeof(double));
    if (kda) orc_kda_spec_rounds_batch(nh, dv, dk, R, S, 0.7, S0, q, k, v, beta, g, acc, os, Ss, 0, NULL, NULL);
    else orc_gdn_spec_rounds_batch(nh, dv, dk, R, S, 0.7, S0, q, k, v, beta, g, acc, os, Ss, 0, NULL, NULL);
    close_to(Ss, ST, (size_t)nh * dv * dk, 1e-12, "delta spec rounds");
    free(S0); free(q); free(k); free(v); free(beta); free(g); free(o); free(ST); free(sn);
    free(orr); free(r); free(acc); free(os); free(Ss);
}

int main(void) {
    orc_set_threads(2);
    mamba2(16, 16, 8, 4);
    mamba2(5, 7, 10, 5);   /* odd sizes */
    mamba2(3, 2, 2, 1);    /* one-entry window */
    delta(0, 16, 8, 8, 4);
    delta(0, 7, 5, 6, 3);
    delta(1, 9, 6, 8, 4);
    delta(1, 4, 3, 2, 1);
    printf("oracle sanitizer run: %d failures\n", fails);
    return fails ? 1 : 0;
}
