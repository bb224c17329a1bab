/*
 * ssm_oracle.c -- plain fp64 CPU oracle for the ReplaySSM decode step.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
 * may load or call this code. It shares no source with the HIP library and includes none of its
 * headers; the product path never reaches it.
 *
 * Pages cited (all carry the title "ReplaySSM: Rethinking State Storage for Faster Hybrid-Model
 * Decoding"):
 *   [feed]      babnews.org feed excerpt (names Mamba-2, Gated DeltaNet and KDA as the SSM layers)
 *   [news]      deskofai.com news article; "para n" = n-th body paragraph
 *   [explainer] nexus-ai-blog.com article; cited by section heading
 * The pages only name the layer types; their recurrences are the published definitions:
 *   Mamba-2: Dao & Gu, "Transformers are SSMs" (ICML 2024), the SSD recurrence with a scalar
 *            (times identity) state matrix per head: h_t = exp(dt_t A) h_{t-1} + dt_t x_t B_t^T,
 *            y_t = h_t C_t + D x_t.
 *   GDN:     Yang, Kautz & Hatamizadeh, "Gated Delta Networks" (ICLR 2025), the gated delta rule:
 *            S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t q_t.
 *   KDA:     Kimi Delta Attention (Kimi Linear, Moonshot AI 2025), the gated delta rule with a
 *            per-key-channel decay: S_t = S_{t-1} D_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *            D_t = diag(exp(g_t)), o_t = S_t q_t.
 *
 * Everything is fp64, one (sequence, head) at a time, in the order the definitions state. The
 * *_batch wrappers only loop over independent heads (OpenMP across heads, nothing inside a head).
 *
 * Layouts (row-major, last index fastest):
 *   Mamba-2 state h [P][N]; inputs x [T][P], B [T][N], C [T][N], dt [T]; output y [T][P].
 *   GDN state S [dv][dk]; inputs q,k [T][dk], v [T][dv], beta [T], g [T] (log-decay); out o [T][dv].
 *   KDA as GDN with g [T][dk] (one log-decay per key channel).
 * snap_after: ascending token counts t (1-based) after which the state is copied into snaps.
 */
#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

static double dotd(const double *a, const double *b, int n) {
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += a[i] * b[i];
    return s;
}

/* ---------------------------------------------------------------------------------------------
 * Mamba-2 sequential recurrence (the definition; the conventional decode step rewrites the state
 * every token -- [news] para 3; [explainer] "Why Decoding, Not Prefill, Is the Hard Part").
 * ------------------------------------------------------------------------------------------- */
void orc_m2_sequential(int P, int N, int T, double A, double D, const double *h0,
                       const double *x, const double *Bm, const double *Cm, const double *dt,
                       double *y, double *h_out, int nsnap, const int *snap_after, double *snaps) {
    size_t sz = (size_t)P * N;
    double *h = (double *)malloc(sz * sizeof(double));
    if (h0) memcpy(h, h0, sz * sizeof(double));
    else memset(h, 0, sz * sizeof(double));
    int si = 0;
    for (int t = 0; t < T; ++t) {
        const double a = exp(dt[t] * A);
        const double *xt = x + (size_t)t * P, *Bt = Bm + (size_t)t * N, *Ct = Cm + (size_t)t * N;
        for (int p = 0; p < P; ++p) {
            double *row = h + (size_t)p * N;
            const double dx = dt[t] * xt[p];
            for (int n = 0; n < N; ++n) row[n] = a * row[n] + dx * Bt[n];
            if (y) y[(size_t)t * P + p] = dotd(row, Ct, N) + D * xt[p];
        }
        while (snaps && si < nsnap && snap_after[si] == t + 1) {
            memcpy(snaps + (size_t)si * sz, h, sz * sizeof(double));
            ++si;
        }
    }
    if (h_out) memcpy(h_out, h, sz * sizeof(double));
    free(h);
}

void orc_m2_sequential_batch(int nh, int P, int N, int T, const double *A, const double *D,
                             const double *h0, const double *x, const double *Bm,
                             const double *Cm, const double *dt, double *y, double *h_out,
                             int nsnap, const int *snap_after, double *snaps) {
    const size_t sz = (size_t)P * N;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nh; ++i) {
        orc_m2_sequential(P, N, T, A[i], D[i], h0 ? h0 + i * sz : NULL,
                          x + (size_t)i * T * P, Bm + (size_t)i * T * N, Cm + (size_t)i * T * N,
                          dt + (size_t)i * T, y ? y + (size_t)i * T * P : NULL,
                          h_out ? h_out + i * sz : NULL, nsnap, snap_after,
                          snaps ? snaps + (size_t)i * nsnap * sz : NULL);
    }
}

/* ---------------------------------------------------------------------------------------------
 * Mamba-2 replay form of one output ([news] para 2: state kept as a checkpoint plus the recent
 * inputs, outputs computed without a state update). Entries 1..k follow the checkpoint hc; entry
 * k is the current token. Unrolling the recurrence k times:
 *   y_k = e^{s_0} hc C_k + sum_i e^{s_i} dt_i (B_i . C_k) x_i + D x_k,  s_i = A sum_{m=i+1..k} dt_m.
 * The decay exponents are suffix sums of dt (never ratios of products).
 * ------------------------------------------------------------------------------------------- */
void orc_m2_replay_output(int P, int N, int k, double A, double D, const double *hc,
                          const double *x, const double *Bm, const double *Ck, const double *dt,
                          double *y) {
    double *w = (double *)malloc((size_t)(k > 0 ? k : 1) * sizeof(double));
    double suffix = 0.0; /* sum of dt over entries after i */
    for (int i = k - 1; i >= 0; --i) {
        w[i] = exp(A * suffix) * dt[i] * dotd(Bm + (size_t)i * N, Ck, N);
        suffix += dt[i];
    }
    const double e0 = exp(A * suffix);
    for (int p = 0; p < P; ++p) {
        double acc = e0 * dotd(hc + (size_t)p * N, Ck, N);
        for (int i = 0; i < k; ++i) acc += w[i] * x[(size_t)i * P + p];
        y[p] = acc + D * x[(size_t)(k - 1) * P + p];
    }
    free(w);
}

/* Mamba-2 flush form ([news] para 3: the buffered inputs are folded into the checkpoint when the
 * buffer fills): h_new = e^{s_0} hc + sum_{i=1..L} e^{s_i} dt_i x_i B_i^T, with s_i as above for
 * k = L. */
void orc_m2_flush(int P, int N, int L, double A, const double *hc, const double *x,
                  const double *Bm, const double *dt, double *h_new) {
    double *u = (double *)malloc((size_t)(L > 0 ? L : 1) * sizeof(double));
    double suffix = 0.0;
    for (int i = L - 1; i >= 0; --i) {
        u[i] = exp(A * suffix) * dt[i];
        suffix += dt[i];
    }
    const double e0 = exp(A * suffix);
    for (int p = 0; p < P; ++p)
        for (int n = 0; n < N; ++n) {
            double acc = e0 * hc[(size_t)p * N + n];
            for (int i = 0; i < L; ++i) acc += u[i] * x[(size_t)i * P + p] * Bm[(size_t)i * N + n];
            h_new[(size_t)p * N + n] = acc;
        }
    free(u);
}

/* Mamba-2 speculative rounds ([news] para 3: drafts are appended and rejected drafts dropped by a
 * pointer move; [explainer] "Usage examples", example 3: propose drafts, verify, keep the accepted
 * prefix). Definition used here: draft j of round r is evaluated by stepping drafts 1..j from the
 * committed state; then the first accept[r] drafts are committed (stepped into the state).
 * x [R][S][P], B/C [R][S][N], dt [R][S]; y [R][S][P]; snap_after counts committed tokens. */
void orc_m2_spec_rounds(int P, int N, int R, int S, double A, double D, const double *h0,
                        const double *x, const double *Bm, const double *Cm, const double *dt,
                        const int *accept, double *y, double *h_out, int nsnap,
                        const int *snap_after, double *snaps) {
    const size_t sz = (size_t)P * N;
    double *h = (double *)malloc(sz * sizeof(double));
    double *hd = (double *)malloc(sz * sizeof(double));
    if (h0) memcpy(h, h0, sz * sizeof(double));
    else memset(h, 0, sz * sizeof(double));
    int pos = 0, si = 0;
    for (int r = 0; r < R; ++r) {
        const size_t o = (size_t)r * S;
        /* drafts from the committed state */
        orc_m2_sequential(P, N, S, A, D, h, x + o * P, Bm + o * N, Cm + o * N, dt + o,
                          y + o * P, hd, 0, NULL, NULL);
        /* commit the accepted prefix one token at a time */
        for (int j = 0; j < accept[r]; ++j) {
            orc_m2_sequential(P, N, 1, A, D, h, x + (o + j) * P, Bm + (o + j) * N,
                              Cm + (o + j) * N, dt + o + j, NULL, h, 0, NULL, NULL);
            ++pos;
            while (snaps && si < nsnap && snap_after[si] == pos) {
                memcpy(snaps + (size_t)si * sz, h, sz * sizeof(double));
                ++si;
            }
        }
    }
    if (h_out) memcpy(h_out, h, sz * sizeof(double));
    free(hd);
    free(h);
}

void orc_m2_spec_rounds_batch(int nh, int P, int N, int R, int S, const double *A,
                              const double *D, const double *h0, const double *x,
                              const double *Bm, const double *Cm, const double *dt,
                              const int *accept /*[nh][R]*/, double *y, double *h_out, int nsnap,
                              const int *snap_after /*[nh][nsnap]*/, double *snaps) {
    const size_t sz = (size_t)P * N, tok = (size_t)R * S;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nh; ++i) {
        orc_m2_spec_rounds(P, N, R, S, A[i], D[i], h0 ? h0 + i * sz : NULL,
                           x + i * tok * P, Bm + i * tok * N, Cm + i * tok * N, dt + i * tok,
                           accept + (size_t)i * R, y + i * tok * P, h_out ? h_out + i * sz : NULL,
                           nsnap, snap_after + (size_t)i * nsnap,
                           snaps ? snaps + (size_t)i * nsnap * sz : NULL);
    }
}

/* ---------------------------------------------------------------------------------------------
 * Gated DeltaNet sequential recurrence (published gated delta rule; named as an SSM layer in [feed]
 * and [news] para 7). Per token, with alpha_t = exp(g_t):
 *   S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,   o_t = scale S_t q_t.
 * Each row p of S evolves on its own, so the update is written row by row.
 * ------------------------------------------------------------------------------------------- */
void orc_gdn_sequential(int dv, int dk, int T, double scale, const double *S0, const double *q,
                        const double *k, const double *v, const double *beta, const double *g,
                        double *o, double *S_out, int nsnap, const int *snap_after,
                        double *snaps) {
    const size_t sz = (size_t)dv * dk;
    double *S = (double *)malloc(sz * sizeof(double));
    if (S0) memcpy(S, S0, sz * sizeof(double));
    else memset(S, 0, sz * sizeof(double));
    int si = 0;
    for (int t = 0; t < T; ++t) {
        const double alpha = exp(g[t]);
        const double *qt = q + (size_t)t * dk, *kt = k + (size_t)t * dk, *vt = v + (size_t)t * dv;
        for (int p = 0; p < dv; ++p) {
            double *row = S + (size_t)p * dk;
            const double sk = alpha * dotd(row, kt, dk); /* (alpha S_{t-1} k_t)[p] */
            const double u = beta[t] * (vt[p] - sk);
            for (int n = 0; n < dk; ++n) row[n] = alpha * row[n] + u * kt[n];
            if (o) o[(size_t)t * dv + p] = scale * dotd(row, qt, dk);
        }
        while (snaps && si < nsnap && snap_after[si] == t + 1) {
            memcpy(snaps + (size_t)si * sz, S, sz * sizeof(double));
            ++si;
        }
    }
    if (S_out) memcpy(S_out, S, sz * sizeof(double));
    free(S);
}

void orc_gdn_sequential_batch(int nh, int dv, int dk, int T, double scale, const double *S0,
                              const double *q, const double *k, const double *v,
                              const double *beta, const double *g, double *o, double *S_out,
                              int nsnap, const int *snap_after, double *snaps) {
    const size_t sz = (size_t)dv * dk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nh; ++i) {
        orc_gdn_sequential(dv, dk, T, scale, S0 ? S0 + i * sz : NULL, q + (size_t)i * T * dk,
                           k + (size_t)i * T * dk, v + (size_t)i * T * dv, beta + (size_t)i * T,
                           g + (size_t)i * T, o ? o + (size_t)i * T * dv : NULL,
                           S_out ? S_out + i * sz : NULL, nsnap, snap_after,
                           snaps ? snaps + (size_t)i * nsnap * sz : NULL);
    }
}

/* GDN speculative rounds (news, para 3: drafts appended to the buffer, the rejected ones dropped by
 * moving a pointer). Per round: the S drafts' outputs from the committed state, each draft seeing
 * the drafts before it; then the state advances by the first accept[r] drafts only. */
void orc_gdn_spec_rounds(int dv, int dk, int R, int S, double scale, const double *S0,
                         const double *q, const double *k, const double *v, const double *beta,
                         const double *g, const int *accept, double *o, double *S_out, int nsnap,
                         const int *snap_after, double *snaps) {
    const size_t sz = (size_t)dv * dk;
    double *St = (double *)malloc(sz * sizeof(double));
    if (S0) memcpy(St, S0, sz * sizeof(double));
    else memset(St, 0, sz * sizeof(double));
    int pos = 0, si = 0;
    for (int r = 0; r < R; ++r) {
        const size_t t0 = (size_t)r * S;
        /* drafts from the committed state (the state itself is not advanced here) */
        orc_gdn_sequential(dv, dk, S, scale, St, q + t0 * dk, k + t0 * dk, v + t0 * dv,
                           beta + t0, g + t0, o + t0 * dv, NULL, 0, NULL, NULL);
        /* commit the accepted prefix one token at a time */
        for (int j = 0; j < accept[r]; ++j) {
            const size_t t = t0 + j;
            orc_gdn_sequential(dv, dk, 1, scale, St, q + t * dk, k + t * dk, v + t * dv,
                               beta + t, g + t, NULL, St, 0, NULL, NULL);
            ++pos;
            while (snaps && si < nsnap && snap_after[si] == pos) {
                memcpy(snaps + (size_t)si * sz, St, sz * sizeof(double));
                ++si;
            }
        }
    }
    if (S_out) memcpy(S_out, St, sz * sizeof(double));
    free(St);
}

void orc_gdn_spec_rounds_batch(int nh, int dv, int dk, int R, int S, double scale,
                               const double *S0, const double *q, const double *k,
                               const double *v, const double *beta, const double *g,
                               const int *accept /*[nh][R]*/, double *o, double *S_out, int nsnap,
                               const int *snap_after /*[nh][nsnap]*/, double *snaps) {
    const size_t sz = (size_t)dv * dk, tok = (size_t)R * S;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nh; ++i) {
        orc_gdn_spec_rounds(dv, dk, R, S, scale, S0 ? S0 + i * sz : NULL, q + i * tok * dk,
                            k + i * tok * dk, v + i * tok * dv, beta + i * tok, g + i * tok,
                            accept + (size_t)i * R, o + i * tok * dv, S_out ? S_out + i * sz : NULL,
                            nsnap, snap_after + (size_t)i * nsnap,
                            snaps ? snaps + (size_t)i * nsnap * sz : NULL);
    }
}

/* ---------------------------------------------------------------------------------------------
 * Kimi Delta Attention sequential recurrence (named as an SSM layer in [feed] and [news] para 7;
 * the published KDA form, the gated delta rule with a per-key-channel decay). Per token, with
 * alpha_t = exp(g_t) a dk-vector (D_t = diag(alpha_t)):
 *   S_t = S_{t-1} D_t + beta_t (v_t - S_{t-1} D_t k_t) k_t^T,   o_t = scale S_t q_t.
 * Row by row: the decayed row is row[n] * alpha[n]; its product with k gives the prediction.
 * g is [T][dk] here (one decay per key channel).
 * ------------------------------------------------------------------------------------------- */
void orc_kda_sequential(int dv, int dk, int T, double scale, const double *S0, const double *q,
                        const double *k, const double *v, const double *beta, const double *g,
                        double *o, double *S_out, int nsnap, const int *snap_after,
                        double *snaps) {
    const size_t sz = (size_t)dv * dk;
    double *S = (double *)malloc(sz * sizeof(double));
    double *alpha = (double *)malloc((size_t)dk * sizeof(double));
    if (S0) memcpy(S, S0, sz * sizeof(double));
    else memset(S, 0, sz * sizeof(double));
    int si = 0;
    for (int t = 0; t < T; ++t) {
        const double *qt = q + (size_t)t * dk, *kt = k + (size_t)t * dk, *vt = v + (size_t)t * dv;
        for (int n = 0; n < dk; ++n) alpha[n] = exp(g[(size_t)t * dk + n]);
        for (int p = 0; p < dv; ++p) {
            double *row = S + (size_t)p * dk;
            for (int n = 0; n < dk; ++n) row[n] *= alpha[n]; /* S_{t-1} D_t */
            const double u = beta[t] * (vt[p] - dotd(row, kt, dk));
            for (int n = 0; n < dk; ++n) row[n] += u * kt[n];
            if (o) o[(size_t)t * dv + p] = scale * dotd(row, qt, dk);
        }
        while (snaps && si < nsnap && snap_after[si] == t + 1) {
            memcpy(snaps + (size_t)si * sz, S, sz * sizeof(double));
            ++si;
        }
    }
    if (S_out) memcpy(S_out, S, sz * sizeof(double));
    free(alpha);
    free(S);
}

void orc_kda_sequential_batch(int nh, int dv, int dk, int T, double scale, const double *S0,
                              const double *q, const double *k, const double *v,
                              const double *beta, const double *g, double *o, double *S_out,
                              int nsnap, const int *snap_after, double *snaps) {
    const size_t sz = (size_t)dv * dk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nh; ++i) {
        orc_kda_sequential(dv, dk, T, scale, S0 ? S0 + i * sz : NULL, q + (size_t)i * T * dk,
                           k + (size_t)i * T * dk, v + (size_t)i * T * dv, beta + (size_t)i * T,
                           g + (size_t)i * T * dk, o ? o + (size_t)i * T * dv : NULL,
                           S_out ? S_out + i * sz : NULL, nsnap, snap_after,
                           snaps ? snaps + (size_t)i * nsnap * sz : NULL);
    }
}

/* The backward walk shared by the GDN and KDA replay forms: r <- q_k, acc <- 0; for i = k..1:
 * c_i = beta_i (k_i . r), acc += c_i v_i, r <- alpha_i (r - c_i k_i), with alpha_i = exp(g_i) one
 * scalar (GDN, gdim = 1) or one value per key channel (KDA, gdim = dk, elementwise). On return r is
 * the query mapped back to the checkpoint's position and acc the buffered entries' value terms,
 * so the output is o = scale (Sc r + acc). */
static void replay_walk(int dv, int dk, int kk, int gdim, const double *qk, const double *k,
                        const double *v, const double *beta, const double *g, double *r,
                        double *acc) {
    memcpy(r, qk, (size_t)dk * sizeof(double));
    memset(acc, 0, (size_t)dv * sizeof(double));
    for (int i = kk - 1; i >= 0; --i) {
        const double *ki = k + (size_t)i * dk, *vi = v + (size_t)i * dv;
        const double c = beta[i] * dotd(ki, r, dk);
        for (int p = 0; p < dv; ++p) acc[p] += c * vi[p];
        for (int n = 0; n < dk; ++n)
            r[n] = exp(g[(size_t)i * gdim + (gdim > 1 ? n : 0)]) * (r[n] - c * ki[n]);
    }
}

/* KDA replay form of one output (the GDN walk with a per-channel decay): r <- q_k, acc <- 0;
 * for i = k..1: c_i = beta_i (k_i . r), acc += c_i v_i, r <- alpha_i * (r - c_i k_i)
 * (elementwise); o = scale (Sc r + acc). */
void orc_kda_replay_output(int dv, int dk, int kk, double scale, const double *Sc,
                           const double *qk, const double *k, const double *v,
                           const double *beta, const double *g, double *o) {
    double *r = (double *)malloc((size_t)dk * sizeof(double));
    double *acc = (double *)malloc((size_t)dv * sizeof(double));
    replay_walk(dv, dk, kk, dk, qk, k, v, beta, g, r, acc);
    for (int p = 0; p < dv; ++p) o[p] = scale * (dotd(Sc + (size_t)p * dk, r, dk) + acc[p]);
    free(acc);
    free(r);
}

/* The query vector r of the replay forms above (GDN: kda = 0, g [kk]; KDA: kda = 1, g [kk][dk]):
 * the checkpoint enters the output only through scale * Sc r, so a change E of the checkpoint
 * (e.g. its read copy's rounding) changes output p by exactly scale * sum_n E[p][n] r[n]. */
void orc_replay_query(int dv, int dk, int kk, int kda, const double *qk, const double *k,
                      const double *v, const double *beta, const double *g, double *r) {
    double *acc = (double *)malloc((size_t)dv * sizeof(double));
    replay_walk(dv, dk, kk, kda ? dk : 1, qk, k, v, beta, g, r, acc);
    free(acc);
}

/* KDA speculative rounds: as orc_gdn_spec_rounds, with the per-channel recurrence. */
void orc_kda_spec_rounds(int dv, int dk, int R, int S, double scale, const double *S0,
                         const double *q, const double *k, const double *v, const double *beta,
                         const double *g, const int *accept, double *o, double *S_out, int nsnap,
                         const int *snap_after, double *snaps) {
    const size_t sz = (size_t)dv * dk;
    double *St = (double *)malloc(sz * sizeof(double));
    if (S0) memcpy(St, S0, sz * sizeof(double));
    else memset(St, 0, sz * sizeof(double));
    int pos = 0, si = 0;
    for (int r = 0; r < R; ++r) {
        const size_t t0 = (size_t)r * S;
        orc_kda_sequential(dv, dk, S, scale, St, q + t0 * dk, k + t0 * dk, v + t0 * dv,
                           beta + t0, g + t0 * dk, o + t0 * dv, NULL, 0, NULL, NULL);
        for (int j = 0; j < accept[r]; ++j) {
            const size_t t = t0 + j;
            orc_kda_sequential(dv, dk, 1, scale, St, q + t * dk, k + t * dk, v + t * dv,
                               beta + t, g + t * dk, NULL, St, 0, NULL, NULL);
            ++pos;
            while (snaps && si < nsnap && snap_after[si] == pos) {
                memcpy(snaps + (size_t)si * sz, St, sz * sizeof(double));
                ++si;
            }
        }
    }
    if (S_out) memcpy(S_out, St, sz * sizeof(double));
    free(St);
}

void orc_kda_spec_rounds_batch(int nh, int dv, int dk, int R, int S, double scale,
                               const double *S0, const double *q, const double *k,
                               const double *v, const double *beta, const double *g,
                               const int *accept, double *o, double *S_out, int nsnap,
                               const int *snap_after, double *snaps) {
    const size_t sz = (size_t)dv * dk, tok = (size_t)R * S;
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < nh; ++i) {
        orc_kda_spec_rounds(dv, dk, R, S, scale, S0 ? S0 + i * sz : NULL, q + i * tok * dk,
                            k + i * tok * dk, v + i * tok * dv, beta + i * tok, g + i * tok * dk,
                            accept + (size_t)i * R, o + i * tok * dv, S_out ? S_out + i * sz : NULL,
                            nsnap, snap_after + (size_t)i * nsnap,
                            snaps ? snaps + (size_t)i * nsnap * sz : NULL);
    }
}

/* GDN replay form of one output: walking the buffered entries from the newest back to the
 * checkpoint, each delta-rule step maps the query through (I - beta k k^T) alpha and emits a
 * value term.  r <- q_k, acc <- 0; for i = k..1: c_i = beta_i (k_i . r), acc += c_i v_i,
 * r <- alpha_i (r - c_i k_i).  Output: o = scale (Sc r + acc). */
void orc_gdn_replay_output(int dv, int dk, int kk, double scale, const double *Sc,
                           const double *qk, const double *k, const double *v,
                           const double *beta, const double *g, double *o) {
    double *r = (double *)malloc((size_t)dk * sizeof(double));
    double *acc = (double *)malloc((size_t)dv * sizeof(double));
    replay_walk(dv, dk, kk, 1, qk, k, v, beta, g, r, acc);
    for (int p = 0; p < dv; ++p) o[p] = scale * (dotd(Sc + (size_t)p * dk, r, dk) + acc[p]);
    free(acc);
    free(r);
}

/* GDN flush in UT/WY form: fold L buffered delta-rule updates into Sc in one pass.
 * With G_t = sum_{m<=t} g_m (log of the cumulative decay gamma_t):
 *   Lm[t][i] = beta_t exp(G_t - G_i) (k_t . k_i) for i < t   (decay as a partial sum of g)
 *   solve (I + Lm) U = diag(beta) V and (I + Lm) W = diag(beta gamma) K by forward substitution
 *   Delta_t = U_t - Sc W_t
 *   S_new = gamma_L Sc + sum_t (gamma_L / gamma_t) Delta_t k_t^T.
 * This is the sequential recurrence regrouped; every decay ratio is an exp of a partial sum. */
void orc_gdn_flush(int dv, int dk, int L, const double *Sc, const double *k, const double *v,
                   const double *beta, const double *g, double *S_new) {
    if (L <= 0) { /* nothing buffered: the checkpoint is unchanged */
        memcpy(S_new, Sc, (size_t)dv * dk * sizeof(double));
        return;
    }
    double *Lm = (double *)calloc((size_t)L * L, sizeof(double));
    double *U = (double *)malloc((size_t)L * dv * sizeof(double));
    double *W = (double *)malloc((size_t)L * dk * sizeof(double));
    double *G = (double *)malloc((size_t)L * sizeof(double));
    double run = 0.0;
    for (int t = 0; t < L; ++t) { run += g[t]; G[t] = run; }
    for (int t = 0; t < L; ++t)
        for (int i = 0; i < t; ++i) {
            double part = 0.0; /* sum_{m=i+1..t} g_m */
            for (int m = i + 1; m <= t; ++m) part += g[m];
            Lm[t * L + i] = beta[t] * exp(part) * dotd(k + (size_t)t * dk, k + (size_t)i * dk, dk);
        }
    for (int t = 0; t < L; ++t) {
        const double gam = exp(G[t]);
        for (int p = 0; p < dv; ++p) {
            double s = beta[t] * v[(size_t)t * dv + p];
            for (int i = 0; i < t; ++i) s -= Lm[t * L + i] * U[(size_t)i * dv + p];
            U[(size_t)t * dv + p] = s;
        }
        for (int n = 0; n < dk; ++n) {
            double s = beta[t] * gam * k[(size_t)t * dk + n];
            for (int i = 0; i < t; ++i) s -= Lm[t * L + i] * W[(size_t)i * dk + n];
            W[(size_t)t * dk + n] = s;
        }
    }
    const double gL = exp(G[L - 1]);
    double *Delta = (double *)malloc((size_t)L * dv * sizeof(double));
    for (int t = 0; t < L; ++t)
        for (int p = 0; p < dv; ++p)
            Delta[(size_t)t * dv + p] =
                U[(size_t)t * dv + p] - dotd(Sc + (size_t)p * dk, W + (size_t)t * dk, dk);
    double *dec = (double *)malloc((size_t)L * sizeof(double));
    for (int t = 0; t < L; ++t) {
        double tail = 0.0; /* log(gamma_L / gamma_t) = sum_{m=t+1..L} g_m */
        for (int m = t + 1; m < L; ++m) tail += g[m];
        dec[t] = exp(tail);
    }
    for (int p = 0; p < dv; ++p)
        for (int n = 0; n < dk; ++n) {
            double acc = gL * Sc[(size_t)p * dk + n];
            for (int t = 0; t < L; ++t)
                acc += dec[t] * Delta[(size_t)t * dv + p] * k[(size_t)t * dk + n];
            S_new[(size_t)p * dk + n] = acc;
        }
    free(dec);
    free(Delta);
    free(G);
    free(W);
    free(U);
    free(Lm);
}

/* Threads of the OpenMP loops over heads (timing only; results do not depend on it). */
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
