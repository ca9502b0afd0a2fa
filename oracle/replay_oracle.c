/*
 * replay_oracle.c -- fp64 CPU oracle for the batched SSM decode step served
 * from a checkpoint plus a buffer of recent per-token records.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark load this library.  It shares no
 * code, header or constant with the GPU path.
 *
 * Everything here is plain loops in double precision, written so that each
 * line can be checked against the formulas on the pages:
 *
 *   [blog]  "ReplaySSM: an SSM decoder that writes its state once every 16
 *           tokens" (ai.thesatyajit.com), sections "Why a fixed-size state is
 *           not cheap to decode", "The identity", "Output without a state",
 *           "The delta-rule wrinkle".
 *   [pr]    vLLM pull request "[Kernel] ReplaySSM: cache SSM inputs for faster
 *           Gated DeltaNet standard decode", sections "Core concept",
 *           "CUDA graphs and continuous batching", and the reviewer's comment
 *           giving S_{t-1} q_t and S_{t-1} k_t from checkpoint plus buffer.
 *
 * Notation.  One tile is one (request row, head).  Its state S is d_v x d_k,
 * stored row-major: S[i*d_k + c].  A token brings v (d_v), k (d_k), q (d_k),
 * a log-decay lam (alpha = exp(lam), alpha in (0,1]) and, for Gated DeltaNet,
 * a write strength beta.  Output o = S_t q_t has d_v entries.
 *
 * Buffer convention (the pages leave it to the reader; this is the plainest
 * reading of [pr] "CUDA graphs and continuous batching" and [blog] "The
 * identity"): a tile holds w records, w = 0..L-1, for the tokens since its
 * checkpoint.  The current token is never read from the buffer.  A non-flush
 * step stores the current token as record w; a flush step folds the w records
 * and the current token into the checkpoint and leaves w = 0.
 *
 * Decay weights are formed as PRODUCTS of alpha, exactly as the pages write
 * gamma_{i:j} = prod alpha_l.  (The GPU path forms them differently.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OC_MAMBA2 = 0, OC_GDN = 1 };

int oc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

static double dot(const double* a, const double* b, int n) {
    double s = 0.0;
    for (int c = 0; c < n; ++c) s += a[c] * b[c];
    return s;
}

/* y = S x for a d_v x d_k row-major S. */
static void matvec(const double* S, const double* x, int dv, int dk, double* y) {
    for (int i = 0; i < dv; ++i) y[i] = dot(S + (int64_t)i * dk, x, dk);
}

/*
 * Conventional decode step, one token per tile, state updated in place.
 *
 * Mamba-2 form ([blog] "Why a fixed-size state is not cheap to decode"):
 *     S_t = alpha_t S_{t-1} + v_t k_t^T,    o_t = S_t q_t.
 * Gated DeltaNet form ([blog] "The delta-rule wrinkle"; [pr] "Core concept"):
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *         = alpha_t S_{t-1} + d_t k_t^T,   d_t = beta_t (v_t - alpha_t S_{t-1} k_t),
 *     o_t = S_t q_t.
 *
 * Arrays: S [n][dv][dk]; q, k [n][dk]; v, out [n][dv]; lam, beta [n]
 * (beta ignored for Mamba-2, may be NULL).  active [n] may be NULL (= all);
 * inactive tiles are left untouched.  xout [n][dv], if not NULL, receives
 * the value written into the state this step (v, or the corrected d).
 */
void oc_conventional_step(int form, int64_t n, int dv, int dk, double* S,
                          const double* q, const double* k, const double* v,
                          const double* lam, const double* beta,
                          const uint8_t* active, double* out, double* xout) {
#pragma omp parallel
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)dv);
        double* d = (double*)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < n; ++t) {
            if (active && !active[t]) continue;
            double* St = S + t * (int64_t)dv * dk;
            const double* qt = q + t * dk;
            const double* kt = k + t * dk;
            const double* vt = v + t * dv;
            const double alpha = exp(lam[t]);
            if (form == OC_GDN) {
                matvec(St, kt, dv, dk, a);                   /* a = S_{t-1} k_t */
                for (int i = 0; i < dv; ++i)
                    d[i] = beta[t] * (vt[i] - alpha * a[i]); /* corrected value */
            } else {
                for (int i = 0; i < dv; ++i) d[i] = vt[i];
            }
            for (int i = 0; i < dv; ++i)
                for (int c = 0; c < dk; ++c)
                    St[(int64_t)i * dk + c] = alpha * St[(int64_t)i * dk + c] + d[i] * kt[c];
            matvec(St, qt, dv, dk, out + t * dv);            /* o_t = S_t q_t */
            if (xout) memcpy(xout + t * dv, d, sizeof(double) * (size_t)dv);
        }
        free(a);
        free(d);
    }
}

/*
 * prod_{l=from..to} alpha_l over a 1-indexed list alpha[1..], empty product = 1.
 * This is the pages' gamma_{from:to}.
 */
static double gamma_range(const double* alpha1, int from, int to) {
    double g = 1.0;
    for (int l = from; l <= to; ++l) g *= alpha1[l];
    return g;
}

/*
 * Replay (checkpoint + buffer) decode step, one token per tile.
 *
 * Per tile: checkpoint C [dv][dk]; buffer of `cap` slots holding w records,
 * record j (0-based) = (lam_j, x_j [dv], k_j [dk]); x = v for Mamba-2 and
 * x = d (the corrected value) for Gated DeltaNet.  flush [n] is the step's
 * flush decision.  w [n] is read and updated: 0 after a flush, w+1 otherwise.
 * Returns the number of tiles whose buffer would overflow (w >= cap on a
 * non-flush step); those tiles are left untouched.
 *
 * Mamba-2 ([blog] "The identity", "Output without a state"): with the w
 * records and the current token numbered j = 1..h, h = w + 1,
 *     S_t = gamma_h C + sum_{j=1..h} gamma_{j+1:h} v_j k_j^T
 *     o_t = gamma_h C q_t + sum_{j=1..h} gamma_{j+1:h} v_j (k_j^T q_t)
 * A flush writes S_t back as the new checkpoint and empties the buffer.
 *
 * Gated DeltaNet ([pr] reviewer comment on the output-only route): with the
 * w records numbered j = 1..w,
 *     S_{t-1} q_t = T (C q_t) + sum_j r_j (k_j . q_t) d_j
 *     S_{t-1} k_t = T (C k_t) + sum_j r_j (k_j . k_t) d_j
 * where T = gamma_{1:w} and r_j = gamma_{j+1:w}.  Then, as in the
 * conventional step, d_t = beta (v - alpha S_{t-1} k_t) and
 * o_t = S_t q_t = alpha S_{t-1} q_t + d_t (k_t . q_t).
 * A flush writes S_t = alpha S_{t-1} + d_t k_t^T with S_{t-1} expanded as
 * T C + sum_j r_j d_j k_j^T.
 */
int64_t oc_replay_step(int form, int64_t n, int dv, int dk, int cap, double* C,
                       double* rec_lam, double* rec_x, double* rec_k, int32_t* w,
                       const uint8_t* flush, const double* q, const double* k,
                       const double* v, const double* lam, const double* beta,
                       const uint8_t* active, double* out) {
    int64_t overflow = 0;
#pragma omp parallel reduction(+ : overflow)
    {
        /* 1-indexed scratch: alpha1[1..h], dots[1..h] */
        double* alpha1 = (double*)malloc(sizeof(double) * (size_t)(cap + 2));
        double* dotq = (double*)malloc(sizeof(double) * (size_t)(cap + 2));
        double* dotk = (double*)malloc(sizeof(double) * (size_t)(cap + 2));
        double* cq = (double*)malloc(sizeof(double) * (size_t)dv);
        double* ck = (double*)malloc(sizeof(double) * (size_t)dv);
        double* d = (double*)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < n; ++t) {
            if (active && !active[t]) continue;
            const int wt = w[t];
            if (!flush[t] && wt >= cap) { overflow += 1; continue; }
            double* Ct = C + t * (int64_t)dv * dk;
            double* lamt = rec_lam + t * (int64_t)cap;
            double* xt = rec_x + t * (int64_t)cap * dv;
            double* kt_rec = rec_k + t * (int64_t)cap * dk;
            const double* qt = q + t * dk;
            const double* kt = k + t * dk;
            const double* vt = v + t * dv;
            const double alpha = exp(lam[t]);
            double* ot = out + t * dv;
            const double kq = dot(kt, qt, dk);

            for (int j = 1; j <= wt; ++j) {
                alpha1[j] = exp(lamt[j - 1]);
                dotq[j] = dot(kt_rec + (int64_t)(j - 1) * dk, qt, dk);
                dotk[j] = dot(kt_rec + (int64_t)(j - 1) * dk, kt, dk);
            }
            matvec(Ct, qt, dv, dk, cq);

            if (form == OC_MAMBA2) {
                const int h = wt + 1;
                alpha1[h] = alpha; /* the current token is position h */
                const double gh = gamma_range(alpha1, 1, h);
                for (int i = 0; i < dv; ++i) {
                    double o = gh * cq[i];
                    for (int j = 1; j <= wt; ++j)
                        o += gamma_range(alpha1, j + 1, h) * xt[(int64_t)(j - 1) * dv + i] * dotq[j];
                    o += vt[i] * kq; /* j = h: gamma_{h+1:h} = 1 */
                    ot[i] = o;
                }
                if (flush[t]) {
                    for (int i = 0; i < dv; ++i)
                        for (int c = 0; c < dk; ++c) {
                            double s = gh * Ct[(int64_t)i * dk + c];
                            for (int j = 1; j <= wt; ++j)
                                s += gamma_range(alpha1, j + 1, h) * xt[(int64_t)(j - 1) * dv + i] *
                                     kt_rec[(int64_t)(j - 1) * dk + c];
                            s += vt[i] * kt[c];
                            Ct[(int64_t)i * dk + c] = s;
                        }
                    w[t] = 0;
                } else {
                    lamt[wt] = lam[t];
                    memcpy(xt + (int64_t)wt * dv, vt, sizeof(double) * (size_t)dv);
                    memcpy(kt_rec + (int64_t)wt * dk, kt, sizeof(double) * (size_t)dk);
                    w[t] = wt + 1;
                }
            } else {
                const double T = gamma_range(alpha1, 1, wt);
                matvec(Ct, kt, dv, dk, ck);
                for (int i = 0; i < dv; ++i) {
                    double sq = T * cq[i]; /* S_{t-1} q_t */
                    double sk = T * ck[i]; /* S_{t-1} k_t */
                    for (int j = 1; j <= wt; ++j) {
                        const double r = gamma_range(alpha1, j + 1, wt);
                        const double dj = xt[(int64_t)(j - 1) * dv + i];
                        sq += r * dotq[j] * dj;
                        sk += r * dotk[j] * dj;
                    }
                    d[i] = beta[t] * (vt[i] - alpha * sk);
                    ot[i] = alpha * sq + d[i] * kq;
                }
                if (flush[t]) {
                    for (int i = 0; i < dv; ++i)
                        for (int c = 0; c < dk; ++c) {
                            double s = T * Ct[(int64_t)i * dk + c];
                            for (int j = 1; j <= wt; ++j)
                                s += gamma_range(alpha1, j + 1, wt) * xt[(int64_t)(j - 1) * dv + i] *
                                     kt_rec[(int64_t)(j - 1) * dk + c];
                            Ct[(int64_t)i * dk + c] = alpha * s + d[i] * kt[c];
                        }
                    w[t] = 0;
                } else {
                    lamt[wt] = lam[t];
                    memcpy(xt + (int64_t)wt * dv, d, sizeof(double) * (size_t)dv);
                    memcpy(kt_rec + (int64_t)wt * dk, kt, sizeof(double) * (size_t)dk);
                    w[t] = wt + 1;
                }
            }
        }
        free(alpha1);
        free(dotq);
        free(dotk);
        free(cq);
        free(ck);
        free(d);
    }
    return overflow;
}

/*
 * Fold the w buffered records of each selected tile into its checkpoint, with
 * no new token ([blog] "The identity" with h = w):
 *     C <- gamma_{1:w} C + sum_{j=1..w} gamma_{j+1:w} x_j k_j^T,   w <- 0.
 * Both forms store records whose state update is S_j = alpha_j S_{j-1} + x_j k_j^T,
 * so the fold is the same for both.  This is the forced, token-less flush a
 * server needs before it retires or preempts a row, or at a prefix-cache
 * block boundary ([pr] "What this PR adds", prefix caching).
 */
void oc_replay_fold(int64_t n, int dv, int dk, int cap, double* C, const double* rec_lam,
                    const double* rec_x, const double* rec_k, int32_t* w, const uint8_t* mask) {
#pragma omp parallel
    {
        double* alpha1 = (double*)malloc(sizeof(double) * (size_t)(cap + 2));
#pragma omp for schedule(static)
        for (int64_t t = 0; t < n; ++t) {
            if (mask && !mask[t]) continue;
            const int wt = w[t];
            double* Ct = C + t * (int64_t)dv * dk;
            const double* xt = rec_x + t * (int64_t)cap * dv;
            const double* kt_rec = rec_k + t * (int64_t)cap * dk;
            for (int j = 1; j <= wt; ++j) alpha1[j] = exp(rec_lam[t * (int64_t)cap + j - 1]);
            const double gw = gamma_range(alpha1, 1, wt);
            for (int i = 0; i < dv; ++i)
                for (int c = 0; c < dk; ++c) {
                    double s = gw * Ct[(int64_t)i * dk + c];
                    for (int j = 1; j <= wt; ++j)
                        s += gamma_range(alpha1, j + 1, wt) * xt[(int64_t)(j - 1) * dv + i] *
                             kt_rec[(int64_t)(j - 1) * dk + c];
                    Ct[(int64_t)i * dk + c] = s;
                }
            w[t] = 0;
        }
        free(alpha1);
    }
}

/*
 * Buffer cursor over a run of decode steps for one row, simulated by counting
 * the records held ([pr] "CUDA graphs and continuous batching": a row flushes
 * when its write position reaches the last buffer slot, L - 1, or when a flush
 * is forced, e.g. on the step that completes a prefix-cache block).
 *   step s:  flush_s = (w == L - 1) or forced_s;  emits (w, flush_s);
 *            then w = 0 after a flush, else w + 1.
 * forced may be NULL.
 */
void oc_cursor_run(int L, int32_t w0, int64_t n_steps, const uint8_t* forced,
                   int32_t* w_out, uint8_t* flush_out) {
    int32_t w = w0;
    for (int64_t s = 0; s < n_steps; ++s) {
        const int f = (w == L - 1) || (forced && forced[s]);
        w_out[s] = w;
        flush_out[s] = (uint8_t)f;
        w = f ? 0 : w + 1;
    }
}
