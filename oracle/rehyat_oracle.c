/*
 * rehyat_oracle.c -- plain fp64 CPU oracle for ReHyAt chunk-wise hybrid attention.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the CPU-baseline
 * leg of the benchmark, never by the product path.  It shares no code with the HIP
 * library.  Slow on purpose: straight loops in the order the method is described,
 * OpenMP only over independent (batch, head) slabs or output rows.
 *
 * Sources (the ReHyAt pages):
 *   [blog]  "ReHyAt (Recurrent Hybrid Attention)" blog post, maplevalley.com.cn:
 *           2.1.1 softmax attention with exp(q.k/sqrt(D)); 2.2.1 hybrid split into a
 *           local softmax region T_S (current chunk plus To overlap frames) and a
 *           linear region T_L (the rest), output = (softmax part + linear part) /
 *           (softmax normaliser + linear normaliser); 2.2.2 phi = grouped 1x1 linear,
 *           split into P parts, each part raised to powers 1..P, concatenated;
 *           2.3 causality across chunks, states S = sum phi(K)^T V, Z = sum phi(K),
 *           S_{t+1} = S_t + sum phi_K V^T, Z_{t+1} = Z_t + sum phi_K;
 *           5.2 streaming loop: the state is carried from chunk to chunk.
 *   [summary] mind-verse.de summary, "Temporaer segmentierte hybride Aufmerksamkeit"
 *           (softmax inside chunks, linear for all other tokens, overlapping chunks) and
 *           "Rekurrente Formulierung" (the hybrid map written as an RNN).
 *
 * Readings where the pages leave a step open (each is also listed in the design notes):
 *   - every part gets all powers 1..P, so F = P*Dphi; feature order is
 *     [part0^1 | part0^2 | .. | part0^P | part1^1 | ..]; parts are contiguous slices of
 *     the Dphi outputs, the first (Dphi mod P) parts one longer;
 *   - the 1x1 linear is followed by softplus (the feature map must stay positive);
 *     bias optional; separate maps for queries and keys, one per head;
 *   - attention inside the softmax window is bidirectional; causality is across chunks;
 *   - T_S = frames [max(0, f0-To), f1) of chunk [f0, f1); T_L = frames [0, max(0, f0-To));
 *     the two regions are disjoint; the last chunk may be shorter than Tc;
 *   - linear_only: T_S empty and T_L = frames [0, f1) (chunk-causal normalised linear
 *     attention), the "empty softmax window" reduction.
 */
#include "rehyat_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- chunk schedule: [blog] 2.2.1 (chunks of Tc frames, To overlap frames), 2.3 ---- */
int orc_schedule(const orc_params* p, int* sched) {
    int nc = (p->T + p->Tc - 1) / p->Tc;
    if (sched) {
        for (int c = 0; c < nc; ++c) {
            int f0 = c * p->Tc;
            int f1 = f0 + p->Tc < p->T ? f0 + p->Tc : p->T;
            int ws, we, ls;
            if (p->linear_only) {
                ws = f1; we = f1; ls = f1;
            } else {
                ws = f0 - p->To > 0 ? f0 - p->To : 0;
                we = f1;
                ls = ws;
            }
            sched[c * 5 + 0] = f0;
            sched[c * 5 + 1] = f1;
            sched[c * 5 + 2] = ws;
            sched[c * 5 + 3] = we;
            sched[c * 5 + 4] = ls;
        }
    }
    return nc;
}

int orc_features(const orc_params* p) { return p->P * p->Dphi; }

static double softplus(double x) {
    /* log(1 + e^x), written so that neither branch overflows */
    return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x)));
}

/* ---- phi: [blog] 2.2.2 -------------------------------------------------------------
 * u = softplus(W x + b)  (one Dphi x D map per head);
 * split u into P contiguous parts; part pi contributes u_pi^1, u_pi^2, .., u_pi^P. */
void orc_phi_head(const orc_params* p, const double* w_h, const double* b_h,
                  const double* x, int64_t count, double* feat) {
    const int D = p->D, Dphi = p->Dphi, P = p->P, F = P * Dphi;
    double* u = (double*)malloc(sizeof(double) * Dphi);
    for (int64_t t = 0; t < count; ++t) {
        const double* xt = x + t * D;
        for (int j = 0; j < Dphi; ++j) {
            double acc = b_h ? b_h[j] : 0.0;
            for (int d = 0; d < D; ++d) acc += w_h[(int64_t)j * D + d] * xt[d];
            u[j] = softplus(acc);
        }
        double* ft = feat + t * F;
        int start = 0, out = 0;
        for (int part = 0; part < P; ++part) {
            int len = Dphi / P + (part < Dphi % P ? 1 : 0);
            for (int pw = 1; pw <= P; ++pw)
                for (int j = start; j < start + len; ++j) ft[out++] = pow(u[j], pw);
            start += len;
        }
    }
    free(u);
}

void orc_phi(const orc_params* p, const double* x, const double* w, const double* bias,
             double* feat) {
    const int64_t N = (int64_t)p->T * p->n;
    const int F = orc_features(p);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < p->B; ++b)
        for (int h = 0; h < p->H; ++h) {
            const int64_t bh = (int64_t)b * p->H + h;
            orc_phi_head(p, w + (int64_t)h * p->Dphi * p->D, bias ? bias + (int64_t)h * p->Dphi : NULL,
                         x + bh * N * p->D, N, feat + bh * N * F);
        }
}

static double dot(const double* a, const double* b, int len) {
    double s = 0.0;
    for (int i = 0; i < len; ++i) s += a[i] * b[i];
    return s;
}

/* Final merge of the two parts for one query ([blog] 2.2.1: shared normaliser).
 * Both numerator and denominator are scaled by exp(-M), M = max(m, 0), which cancels. */
static void merge(int D, int has_soft, double m, double l, const double* num, int has_lin,
                  const double* y, double z, double* out) {
    double M = has_soft ? (m > 0 ? m : 0.0) : 0.0;
    double a = has_soft ? exp(m - M) : 0.0;
    double g = has_lin ? exp(-M) : 0.0;
    double den = a * l + g * z;
    for (int d = 0; d < D; ++d) out[d] = (a * (has_soft ? num[d] : 0.0) + g * (has_lin ? y[d] : 0.0)) / den;
}

/* Softmax part of one query over keys [k0, k1) of one (b,h) slab: max m, sum l,
 * unnormalised numerator num = sum exp(s - m) v. */
static void softmax_part(int D, const double* qi, const double* kbh, const double* vbh,
                         int64_t k0, int64_t k1, double* m, double* l, double* num) {
    const double scale = 1.0 / sqrt((double)D);
    double mx = -INFINITY;
    for (int64_t j = k0; j < k1; ++j) {
        double s = dot(qi, kbh + j * D, D) * scale;
        if (s > mx) mx = s;
    }
    double sum = 0.0;
    for (int d = 0; d < D; ++d) num[d] = 0.0;
    for (int64_t j = k0; j < k1; ++j) {
        double e = exp(dot(qi, kbh + j * D, D) * scale - mx);
        sum += e;
        for (int d = 0; d < D; ++d) num[d] += e * vbh[j * D + d];
    }
    *m = mx;
    *l = sum;
}

static void write_aux(int D, int64_t row, int has_soft, double m, double l, const double* num,
                      const double* y, double z, double* osoft, double* lse, double* ya,
                      double* za) {
    if (osoft)
        for (int d = 0; d < D; ++d) osoft[row * D + d] = has_soft ? num[d] / l : 0.0;
    if (lse) lse[row] = has_soft ? m + log(l) : -INFINITY;
    if (ya)
        for (int d = 0; d < D; ++d) ya[row * D + d] = y[d];
    if (za) za[row] = z;
}

/* ---- brute force: the definition, O(N^2) per slab ----------------------------------
 * For query i in chunk c: T_S = tokens of frames [ws, we), T_L = tokens of frames [0, ls);
 * o_i = (sum_{T_S} e^{q.k/sqrt D} v + sum_{T_L} kappa v) / (sum_{T_S} e^{q.k/sqrt D} + sum_{T_L} kappa),
 * kappa = phi_q(q_i) . phi_k(k_j). */
void orc_bruteforce(const orc_params* p, const double* q, const double* k, const double* v,
                    const double* wq, const double* wk, const double* bq, const double* bk,
                    double* out, double* osoft, double* lse, double* y, double* z) {
    const int D = p->D, H = p->H, n = p->n, F = orc_features(p);
    const int64_t N = (int64_t)p->T * n;
    int nc = orc_schedule(p, NULL);
    int* sched = (int*)malloc(sizeof(int) * 5 * nc);
    orc_schedule(p, sched);
    const double scale = 1.0 / sqrt((double)D);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < p->B; ++b)
        for (int h = 0; h < H; ++h) {
            const int64_t base = ((int64_t)b * H + h) * N;
            const double* qbh = q + base * D;
            const double* kbh = k + base * D;
            const double* vbh = v + base * D;
            double* fq = (double*)malloc(sizeof(double) * N * F);
            double* fk = (double*)malloc(sizeof(double) * N * F);
            double* s = (double*)malloc(sizeof(double) * N);
            double* wgt = (double*)malloc(sizeof(double) * N);
            double* num = (double*)malloc(sizeof(double) * D);
            double* yv = (double*)malloc(sizeof(double) * D);
            orc_phi_head(p, wq + (int64_t)h * p->Dphi * D, bq ? bq + (int64_t)h * p->Dphi : NULL, qbh, N, fq);
            orc_phi_head(p, wk + (int64_t)h * p->Dphi * D, bk ? bk + (int64_t)h * p->Dphi : NULL, kbh, N, fk);
            for (int64_t i = 0; i < N; ++i) {
                const int* sc = sched + 5 * ((int)(i / n) / p->Tc);
                const int ws = sc[2], we = sc[3], ls = sc[4];
                int has_soft = we > ws, has_lin = ls > 0;
                /* scores over the softmax region and their max */
                double m = -INFINITY;
                for (int64_t j = 0; j < N; ++j) {
                    int f = (int)(j / n);
                    if (f >= ws && f < we) {
                        s[j] = dot(qbh + i * D, kbh + j * D, D) * scale;
                        if (s[j] > m) m = s[j];
                    }
                }
                /* per-key weights relative to exp(m): softmax keys exp(s-m), linear keys kappa */
                double l = 0.0, zz = 0.0;
                for (int64_t j = 0; j < N; ++j) {
                    int f = (int)(j / n);
                    if (f >= ws && f < we) {
                        wgt[j] = exp(s[j] - m);
                        l += wgt[j];
                    } else if (f < ls) {
                        wgt[j] = dot(fq + i * F, fk + j * F, F);
                        zz += wgt[j];
                    } else {
                        wgt[j] = 0.0;
                    }
                }
                for (int d = 0; d < D; ++d) { num[d] = 0.0; yv[d] = 0.0; }
                for (int64_t j = 0; j < N; ++j) {
                    int f = (int)(j / n);
                    if (wgt[j] == 0.0) continue;
                    double* acc = (f >= ws && f < we) ? num : yv;
                    for (int d = 0; d < D; ++d) acc[d] += wgt[j] * vbh[j * D + d];
                }
                merge(D, has_soft, m, l, num, has_lin, yv, zz, out + (base + i) * D);
                write_aux(D, base + i, has_soft, m, l, num, yv, zz, osoft, lse, y, z);
            }
            free(fq); free(fk); free(s); free(wgt); free(num); free(yv);
        }
    free(sched);
}

/* S += phi_k(k_j)^T v_j and Z += phi_k(k_j) over tokens [t0, t1) ([blog] 2.3 update rule). */
static void absorb(int D, int F, const double* fk, const double* vbh, int64_t t0, int64_t t1,
                   double* S, double* Z) {
    for (int64_t j = t0; j < t1; ++j)
        for (int f = 0; f < F; ++f) {
            double a = fk[j * F + f];
            Z[f] += a;
            for (int d = 0; d < D; ++d) S[(int64_t)f * D + d] += a * vbh[j * D + d];
        }
}

/* One query of chunk c given the linear state (S, Z) that covers T_L. */
static void query_with_state(const orc_params* p, const int* sc, const double* qi,
                             const double* fqi, const double* kbh, const double* vbh,
                             const double* S, const double* Z, int64_t row, double* out,
                             double* osoft, double* lse, double* ya, double* za, double* num,
                             double* yv) {
    const int D = p->D, n = p->n, F = orc_features(p);
    const int ws = sc[2], we = sc[3], ls = sc[4];
    int has_soft = we > ws, has_lin = ls > 0;
    double m = 0.0, l = 0.0, zz = 0.0;
    if (has_soft) softmax_part(D, qi, kbh, vbh, (int64_t)ws * n, (int64_t)we * n, &m, &l, num);
    for (int d = 0; d < D; ++d) yv[d] = 0.0;
    if (has_lin) {
        for (int f = 0; f < F; ++f) {
            zz += fqi[f] * Z[f];
            for (int d = 0; d < D; ++d) yv[d] += fqi[f] * S[(int64_t)f * D + d];
        }
    }
    merge(D, has_soft, m, l, num, has_lin, yv, zz, out + row * D);
    write_aux(D, row, has_soft, m, l, num, yv, zz, osoft, lse, ya, za);
}

/* ---- recurrent form: [blog] 2.3, S and Z carried from chunk to chunk ---------------- */
void orc_recurrent(const orc_params* p, const double* q, const double* k, const double* v,
                   const double* wq, const double* wk, const double* bq, const double* bk,
                   double* out, double* osoft, double* lse, double* y, double* z) {
    const int D = p->D, H = p->H, n = p->n, F = orc_features(p);
    const int64_t N = (int64_t)p->T * n;
    int nc = orc_schedule(p, NULL);
    int* sched = (int*)malloc(sizeof(int) * 5 * nc);
    orc_schedule(p, sched);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < p->B; ++b)
        for (int h = 0; h < H; ++h) {
            const int64_t base = ((int64_t)b * H + h) * N;
            const double* kbh = k + base * D;
            const double* vbh = v + base * D;
            double* fq = (double*)malloc(sizeof(double) * N * F);
            double* fk = (double*)malloc(sizeof(double) * N * F);
            double* S = (double*)calloc((size_t)F * D, sizeof(double));
            double* Z = (double*)calloc((size_t)F, sizeof(double));
            double* num = (double*)malloc(sizeof(double) * D);
            double* yv = (double*)malloc(sizeof(double) * D);
            orc_phi_head(p, wq + (int64_t)h * p->Dphi * D, bq ? bq + (int64_t)h * p->Dphi : NULL, q + base * D, N, fq);
            orc_phi_head(p, wk + (int64_t)h * p->Dphi * D, bk ? bk + (int64_t)h * p->Dphi : NULL, kbh, N, fk);
            int absorbed = 0; /* frames [0, absorbed) are in S, Z */
            for (int c = 0; c < nc; ++c) {
                const int* sc = sched + 5 * c;
                absorb(D, F, fk, vbh, (int64_t)absorbed * n, (int64_t)sc[4] * n, S, Z);
                absorbed = sc[4];
                for (int64_t i = (int64_t)sc[0] * n; i < (int64_t)sc[1] * n; ++i)
                    query_with_state(p, sc, q + (base + i) * D, fq + i * F, kbh, vbh, S, Z, base + i,
                                     out, osoft, lse, y, z, num, yv);
            }
            free(fq); free(fk); free(S); free(Z); free(num); free(yv);
        }
    free(sched);
}

/* Per-chunk partials Delta_c over frames [ls(c-1), ls(c)) and their inclusive prefix
 * S_c = sum_{c' <= c} Delta_c' for one slab.  Sc: [nc, F, D], Zc: [nc, F]. */
static void chunk_states(const orc_params* p, const int* sched, int nc, const double* fk,
                         const double* vbh, double* Sc, double* Zc) {
    const int D = p->D, n = p->n, F = orc_features(p);
    int prev = 0;
    for (int c = 0; c < nc; ++c) {
        double* S = Sc + (int64_t)c * F * D;
        double* Z = Zc + (int64_t)c * F;
        memset(S, 0, sizeof(double) * F * D);
        memset(Z, 0, sizeof(double) * F);
        absorb(D, F, fk, vbh, (int64_t)prev * n, (int64_t)sched[5 * c + 4] * n, S, Z); /* Delta_c */
        prev = sched[5 * c + 4];
    }
    for (int c = 1; c < nc; ++c) { /* prefix sum over chunks */
        for (int64_t e = 0; e < (int64_t)F * D; ++e) Sc[(int64_t)c * F * D + e] += Sc[(int64_t)(c - 1) * F * D + e];
        for (int f = 0; f < F; ++f) Zc[(int64_t)c * F + f] += Zc[(int64_t)(c - 1) * F + f];
    }
}

/* ---- chunk-parallel form: all Delta_c, prefix over chunks, then every chunk at once ---- */
void orc_parallel(const orc_params* p, const double* q, const double* k, const double* v,
                  const double* wq, const double* wk, const double* bq, const double* bk,
                  double* out, double* osoft, double* lse, double* y, double* z) {
    const int D = p->D, H = p->H, n = p->n, F = orc_features(p);
    const int64_t N = (int64_t)p->T * n;
    int nc = orc_schedule(p, NULL);
    int* sched = (int*)malloc(sizeof(int) * 5 * nc);
    orc_schedule(p, sched);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < p->B; ++b)
        for (int h = 0; h < H; ++h) {
            const int64_t base = ((int64_t)b * H + h) * N;
            const double* kbh = k + base * D;
            const double* vbh = v + base * D;
            double* fq = (double*)malloc(sizeof(double) * N * F);
            double* fk = (double*)malloc(sizeof(double) * N * F);
            double* Sc = (double*)malloc(sizeof(double) * nc * F * D);
            double* Zc = (double*)malloc(sizeof(double) * nc * F);
            double* num = (double*)malloc(sizeof(double) * D);
            double* yv = (double*)malloc(sizeof(double) * D);
            orc_phi_head(p, wq + (int64_t)h * p->Dphi * D, bq ? bq + (int64_t)h * p->Dphi : NULL, q + base * D, N, fq);
            orc_phi_head(p, wk + (int64_t)h * p->Dphi * D, bk ? bk + (int64_t)h * p->Dphi : NULL, kbh, N, fk);
            chunk_states(p, sched, nc, fk, vbh, Sc, Zc);
            for (int64_t i = 0; i < N; ++i) {
                int c = (int)(i / n) / p->Tc;
                query_with_state(p, sched + 5 * c, q + (base + i) * D, fq + i * F, kbh, vbh,
                                 Sc + (int64_t)c * F * D, Zc + (int64_t)c * F, base + i, out, osoft,
                                 lse, y, z, num, yv);
            }
            free(fq); free(fk); free(Sc); free(Zc); free(num); free(yv);
        }
    free(sched);
}

static int cmp_i64(const void* a, const void* b) {
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return x < y ? -1 : x > y;
}

void orc_parallel_rows(const orc_params* p, const double* q, const double* k, const double* v,
                       const double* wq, const double* wk, const double* bq, const double* bk,
                       int64_t nrows, const int64_t* rows,
                       double* out, double* osoft, double* lse, double* y, double* z) {
    const int D = p->D, H = p->H, n = p->n, F = orc_features(p);
    const int64_t N = (int64_t)p->T * n;
    int nc = orc_schedule(p, NULL);
    int* sched = (int*)malloc(sizeof(int) * 5 * nc);
    orc_schedule(p, sched);
    /* which slabs are touched */
    int64_t* slabs = (int64_t*)malloc(sizeof(int64_t) * (nrows > 0 ? nrows : 1));
    for (int64_t r = 0; r < nrows; ++r) slabs[r] = rows[r] / N;
    qsort(slabs, (size_t)nrows, sizeof(int64_t), cmp_i64);
    int64_t nslab = 0;
    for (int64_t r = 0; r < nrows; ++r)
        if (nslab == 0 || slabs[nslab - 1] != slabs[r]) slabs[nslab++] = slabs[r];
    for (int64_t si = 0; si < nslab; ++si) {
        const int64_t bh = slabs[si];
        const int h = (int)(bh % H);
        const int64_t base = bh * N;
        const double* kbh = k + base * D;
        const double* vbh = v + base * D;
        double* fk = (double*)malloc(sizeof(double) * N * F);
        double* Sc = (double*)malloc(sizeof(double) * nc * F * D);
        double* Zc = (double*)malloc(sizeof(double) * nc * F);
        /* phi(K) over the whole slab, split over threads by token */
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < N; ++t)
            orc_phi_head(p, wk + (int64_t)h * p->Dphi * D, bk ? bk + (int64_t)h * p->Dphi : NULL,
                         kbh + t * D, 1, fk + t * F);
        chunk_states(p, sched, nc, fk, vbh, Sc, Zc);
#pragma omp parallel for schedule(dynamic)
        for (int64_t r = 0; r < nrows; ++r) {
            if (rows[r] / N != bh) continue;
            const int64_t i = rows[r] % N;
            double* fq = (double*)malloc(sizeof(double) * F);
            double* num = (double*)malloc(sizeof(double) * D);
            double* yv = (double*)malloc(sizeof(double) * D);
            orc_phi_head(p, wq + (int64_t)h * p->Dphi * D, bq ? bq + (int64_t)h * p->Dphi : NULL,
                         q + (base + i) * D, 1, fq);
            int c = (int)(i / n) / p->Tc;
            query_with_state(p, sched + 5 * c, q + (base + i) * D, fq, kbh, vbh,
                             Sc + (int64_t)c * F * D, Zc + (int64_t)c * F, r, out, osoft, lse, y, z,
                             num, yv);
            free(fq); free(num); free(yv);
        }
        free(fk); free(Sc); free(Zc);
    }
    free(slabs);
    free(sched);
}

/* ---- streaming form: [blog] 5.2, one call per chunk with carried states ---------------
 * State (doubles): [frames_seen, frames_absorbed, closed, pad] then per slab
 * S [F,D], Z [F], overlap K [To*n, D], overlap V [To*n, D].  The overlap holds the frames
 * [frames_absorbed, frames_seen) that are still inside the next softmax window. */
static int64_t slab_state(const orc_params* p) {
    const int64_t F = orc_features(p);
    return F * p->D + F + 2 * (int64_t)p->To * p->n * p->D;
}

int64_t orc_stream_state_doubles(const orc_params* p) {
    return 4 + (int64_t)p->B * p->H * slab_state(p);
}

void orc_stream_init(const orc_params* p, double* state) {
    memset(state, 0, sizeof(double) * orc_stream_state_doubles(p));
}

int orc_stream_step(const orc_params* p, double* state, const double* q, const double* k,
                    const double* v, int frames, const double* wq, const double* wk,
                    const double* bq, const double* bk, double* out) {
    const int D = p->D, H = p->H, n = p->n, F = orc_features(p), To = p->To;
    if (frames < 1 || frames > p->Tc || state[2] != 0.0) return -1;
    const int f0 = (int)state[0], f1 = f0 + frames;
    const int absorbed = (int)state[1];
    const int held = f0 - absorbed;                    /* frames in the overlap buffer */
    const int ws = p->linear_only ? f1 : (f0 - To > 0 ? f0 - To : 0);
    const int ls = ws;                                 /* T_L = frames [0, ls) */
    const int next_abs = p->linear_only ? f1 : (f1 - To > 0 ? f1 - To : 0);
    const int64_t Lc = (int64_t)frames * n;
    /* the window is [held overlap frames | this chunk]: local tokens [0, (held+frames)*n) */
    const int64_t Lw = (int64_t)(held + frames) * n;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < p->B; ++b)
        for (int h = 0; h < H; ++h) {
            const int64_t bh = (int64_t)b * H + h;
            double* slab = state + 4 + bh * slab_state(p);
            double* S = slab;
            double* Z = S + (int64_t)F * D;
            double* ok = Z + F;
            double* ov = ok + (int64_t)To * n * D;
            const double* qc = q + bh * Lc * D;
            const double* kc = k + bh * Lc * D;
            const double* vc = v + bh * Lc * D;
            /* window keys/values: overlap frames then chunk frames */
            double* wkey = (double*)malloc(sizeof(double) * (Lw > 0 ? Lw : 1) * D);
            double* wval = (double*)malloc(sizeof(double) * (Lw > 0 ? Lw : 1) * D);
            memcpy(wkey, ok, sizeof(double) * held * n * D);
            memcpy(wval, ov, sizeof(double) * held * n * D);
            memcpy(wkey + (int64_t)held * n * D, kc, sizeof(double) * Lc * D);
            memcpy(wval + (int64_t)held * n * D, vc, sizeof(double) * Lc * D);
            double* fk = (double*)malloc(sizeof(double) * (Lw > 0 ? Lw : 1) * F);
            orc_phi_head(p, wk + (int64_t)h * p->Dphi * D, bk ? bk + (int64_t)h * p->Dphi : NULL, wkey, Lw, fk);
            /* frames [absorbed, ls) enter the state before this chunk reads it
             * (only in linear_only mode, where the chunk itself is linear) */
            absorb(D, F, fk, wval, 0, (int64_t)(ls - absorbed) * n, S, Z);
            /* softmax window = local frames [ws - absorbed, held + frames) */
            int lsc[5] = {0, 0, (ws - absorbed), held + frames, ls};
            if (p->linear_only) { lsc[2] = held + frames; lsc[3] = held + frames; }
            double* fq = (double*)malloc(sizeof(double) * F);
            double* num = (double*)malloc(sizeof(double) * D);
            double* yv = (double*)malloc(sizeof(double) * D);
            double* tmp = (double*)malloc(sizeof(double) * D);
            for (int64_t i = 0; i < Lc; ++i) {
                orc_phi_head(p, wq + (int64_t)h * p->Dphi * D, bq ? bq + (int64_t)h * p->Dphi : NULL, qc + i * D, 1, fq);
                /* query_with_state takes the window in frames of the local key buffer */
                query_with_state(p, lsc, qc + i * D, fq, wkey, wval, S, Z, 0, tmp, NULL, NULL,
                                 NULL, NULL, num, yv);
                memcpy(out + (bh * Lc + i) * D, tmp, sizeof(double) * D);
            }
            /* frames that leave the window enter the state ([blog] 2.3 update) */
            int from = ls > absorbed ? ls : absorbed;
            absorb(D, F, fk, wval, (int64_t)(from - absorbed) * n, (int64_t)(next_abs - absorbed) * n, S, Z);
            /* keep the frames [next_abs, f1) as the new overlap */
            int keep = f1 - next_abs;
            memcpy(ok, wkey + (int64_t)(next_abs - absorbed) * n * D, sizeof(double) * keep * n * D);
            memcpy(ov, wval + (int64_t)(next_abs - absorbed) * n * D, sizeof(double) * keep * n * D);
            free(wkey); free(wval); free(fk); free(fq); free(num); free(yv); free(tmp);
        }
    state[0] = f1;
    state[1] = next_abs;
    if (frames < p->Tc) state[2] = 1.0;
    return 0;
}
