/*
 * rehyat_oracle.h -- plain fp64 CPU oracle for ReHyAt chunk-wise hybrid attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  The product path never calls it and
 * shares no code, header or constant with it.
 *
 * What it computes follows the ReHyAt pages:
 *   - "ReHyAt (Recurrent Hybrid Attention)" blog, maplevalley.com.cn, section 2.2.1
 *     (hybrid split: softmax over the local chunk plus overlap, linear attention over
 *     the rest, one shared normaliser), section 2.2.2 (polynomial feature map phi),
 *     section 2.3 (causality across chunks, states S and Z and their update rule),
 *     section 5.2 (chunk-by-chunk streaming loop with carried states);
 *   - the paper abstract (chatpaper.ai) and the mind-verse.de summary, sections
 *     "Temporaer segmentierte hybride Aufmerksamkeit" and "Rekurrente Formulierung"
 *     (overlapping chunks; the recurrent form is a reformulation of the same map).
 *
 * Every array is row-major float64.  Shapes use:
 *   B batch, H heads, D head dim, T frames, n tokens per frame, N = T*n,
 *   Tc chunk frames, To overlap frames, Dphi phi width, P parts = max power,
 *   F = P*Dphi features.
 *   q, k, v : [B,H,N,D]        wq, wk : [H,Dphi,D]       bq, bk : [H,Dphi] or NULL
 *   out     : [B,H,N,D]
 * Aux outputs (each may be NULL):
 *   osoft [B,H,N,D]  softmax part normalised by its own sum (0 where the window is empty)
 *   lse   [B,H,N]    natural log of the softmax denominator sum_j exp(q.k_j/sqrt(D))
 *                    (-inf where the window is empty)
 *   y     [B,H,N,D]  linear numerator   phi_q(q) . sum_{j in T_L} phi_k(k_j) v_j^T
 *   z     [B,H,N]    linear denominator phi_q(q) . sum_{j in T_L} phi_k(k_j)
 */
#ifndef REHYAT_ORACLE_H
#define REHYAT_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int B, H, D, T, n, Tc, To, Dphi, P, linear_only;
} orc_params;

/* Chunk schedule: returns the number of chunks; fills sched[c*5 + {0..4}] =
 * f0, f1, ws, we, ls (frame indices) when sched != NULL. */
int orc_schedule(const orc_params* p, int* sched);

int orc_features(const orc_params* p);

/* phi for one head over `count` tokens: x [count,D] -> feat [count,F]. */
void orc_phi_head(const orc_params* p, const double* w_h, const double* b_h,
                  const double* x, int64_t count, double* feat);

/* phi over [B,H,N,D] with per-head weights. */
void orc_phi(const orc_params* p, const double* x, const double* w, const double* bias,
             double* feat);

/* O(N^2) masked hybrid formula, the definition. */
void orc_bruteforce(const orc_params* p, const double* q, const double* k, const double* v,
                    const double* wq, const double* wk, const double* bq, const double* bk,
                    double* out, double* osoft, double* lse, double* y, double* z);

/* Recurrent form: states S, Z absorbed chunk after chunk. */
void orc_recurrent(const orc_params* p, const double* q, const double* k, const double* v,
                   const double* wq, const double* wk, const double* bq, const double* bk,
                   double* out, double* osoft, double* lse, double* y, double* z);

/* Chunk-parallel form: per-chunk partial states, prefix sum over chunks, combine. */
void orc_parallel(const orc_params* p, const double* q, const double* k, const double* v,
                  const double* wq, const double* wk, const double* bq, const double* bk,
                  double* out, double* osoft, double* lse, double* y, double* z);

/* Chunk-parallel form evaluated on selected rows only.  rows[i] indexes the flattened
 * [B*H*N] query axis; outputs are packed per selected row: out [nrows,D],
 * osoft [nrows,D], lse [nrows], y [nrows,D], z [nrows].  The states are built in full. */
void orc_parallel_rows(const orc_params* p, const double* q, const double* k, const double* v,
                       const double* wq, const double* wk, const double* bq, const double* bk,
                       int64_t nrows, const int64_t* rows,
                       double* out, double* osoft, double* lse, double* y, double* z);

/* Streaming form: one call per chunk of `frames` frames, state carried between calls.
 * State layout is private to the oracle; size it with orc_stream_state_doubles(). */
int64_t orc_stream_state_doubles(const orc_params* p);
void orc_stream_init(const orc_params* p, double* state);
/* q,k,v: [B,H,frames*n,D] for this chunk; out: [B,H,frames*n,D].  Returns 0 on success,
 * -1 if frames is out of range or the stream was closed by a shorter final chunk. */
int orc_stream_step(const orc_params* p, double* state, const double* q, const double* k,
                    const double* v, int frames, const double* wq, const double* wk,
                    const double* bq, const double* bk, double* out);

#ifdef __cplusplus
}
#endif
#endif
