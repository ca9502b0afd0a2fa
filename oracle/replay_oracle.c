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
 *   [nv]    NVIDIA technical blog "ReplaySSM: Rethinking state storage for
 *           faster hybrid model decoding", section "Benefit 2: Simplify
 *           rollback and speed up verification".
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

/*
 * Speculative verify step, Mamba-2 form ([blog] "Speculative decoding:
 * rollback becomes a pointer"; [nv] "Benefit 2: Simplify rollback and speed
 * up verification").  Per tile: checkpoint C, h committed records
 * j = 1..h (lam_j, x_j, k_j) in slots 0..h-1 of a buffer of `cap` slots, and
 * T draft tokens i = 1..T with (lam^d_i, v_i, k_i, q_i).  The output for
 * draft i is the state after the committed records and drafts 1..i, applied
 * to q_i ([nv]: one read of the checkpoint for all T queries, K^T Q, D the
 * cumulative decays of the draft positions, W a causally masked matrix of
 * decays):
 *     o_i = gamma_{1:h} D_i (C q_i) + sum_{j=1..h} gamma_{j+1:h} D_i (k_j . q_i) x_j
 *         + sum_{m=1..i} W_{im} (k_m . q_i) v_m
 *     D_i = prod_{l=1..i} alpha^d_l,   W_{im} = prod_{l=m+1..i} alpha^d_l (m <= i).
 * flush [n] is decided before acceptance is known; a flushing tile folds
 * only its committed records,
 *     C <- gamma_{1:h} C + sum_j gamma_{j+1:h} x_j k_j^T,   h <- 0,
 * and every tile then stores its T drafts as records in slots h..h+T-1
 * ([blog]: the drafts are appended behind the committed records; records
 * past the committed pointer are ignored and later overwritten).  Accepting
 * drafts is oc_spec_commit.  Inputs: q, k [n][T][dk]; v, out [n][T][dv];
 * lam [n][T].  Returns the number of tiles whose drafts would not fit the
 * ring (h + T > cap without a flush, or T > cap); those tiles are left
 * untouched.
 */
int64_t oc_spec_verify(int64_t n, int dv, int dk, int cap, int T, double* C, double* rec_lam,
                       double* rec_x, double* rec_k, int32_t* h, const uint8_t* flush,
                       const double* q, const double* k, const double* v, const double* lam,
                       const uint8_t* active, double* out) {
    int64_t overflow = 0;
#pragma omp parallel reduction(+ : overflow)
    {
        double* ac = (double*)malloc(sizeof(double) * (size_t)(cap + 2)); /* committed alphas, 1-indexed */
        double* ad = (double*)malloc(sizeof(double) * (size_t)(T + 2));   /* draft alphas, 1-indexed */
        double* cq = (double*)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < n; ++t) {
            if (active && !active[t]) continue;
            const int ht = h[t];
            const int base = flush[t] ? 0 : ht; /* first slot of this step's drafts */
            if (base + T > cap) { overflow += 1; continue; }
            double* Ct = C + t * (int64_t)dv * dk;
            double* lamt = rec_lam + t * (int64_t)cap;
            double* xt = rec_x + t * (int64_t)cap * dv;
            double* krt = rec_k + t * (int64_t)cap * dk;
            const double* qt = q + t * (int64_t)T * dk;
            const double* kt = k + t * (int64_t)T * dk;
            const double* vt = v + t * (int64_t)T * dv;
            const double* lt = lam + t * (int64_t)T;
            double* ot = out + t * (int64_t)T * dv;
            for (int j = 1; j <= ht; ++j) ac[j] = exp(lamt[j - 1]);
            for (int i = 1; i <= T; ++i) ad[i] = exp(lt[i - 1]);
            const double gh = gamma_range(ac, 1, ht);
            for (int i = 1; i <= T; ++i) {
                const double* qi = qt + (int64_t)(i - 1) * dk;
                const double Di = gamma_range(ad, 1, i);
                matvec(Ct, qi, dv, dk, cq);
                for (int r = 0; r < dv; ++r) ot[(int64_t)(i - 1) * dv + r] = gh * Di * cq[r];
                for (int j = 1; j <= ht; ++j) {
                    const double wgt = gamma_range(ac, j + 1, ht) * Di * dot(krt + (int64_t)(j - 1) * dk, qi, dk);
                    for (int r = 0; r < dv; ++r) ot[(int64_t)(i - 1) * dv + r] += wgt * xt[(int64_t)(j - 1) * dv + r];
                }
                for (int m = 1; m <= i; ++m) {
                    const double wgt = gamma_range(ad, m + 1, i) * dot(kt + (int64_t)(m - 1) * dk, qi, dk);
                    for (int r = 0; r < dv; ++r) ot[(int64_t)(i - 1) * dv + r] += wgt * vt[(int64_t)(m - 1) * dv + r];
                }
            }
            if (flush[t]) {
                for (int r = 0; r < dv; ++r)
                    for (int c = 0; c < dk; ++c) {
                        double s = gh * Ct[(int64_t)r * dk + c];
                        for (int j = 1; j <= ht; ++j)
                            s += gamma_range(ac, j + 1, ht) * xt[(int64_t)(j - 1) * dv + r] * krt[(int64_t)(j - 1) * dk + c];
                        Ct[(int64_t)r * dk + c] = s;
                    }
                h[t] = 0;
            }
            for (int i = 0; i < T; ++i) {
                lamt[base + i] = lt[i];
                memcpy(xt + (int64_t)(base + i) * dv, vt + (int64_t)i * dv, sizeof(double) * (size_t)dv);
                memcpy(krt + (int64_t)(base + i) * dk, kt + (int64_t)i * dk, sizeof(double) * (size_t)dk);
            }
        }
        free(ac);
        free(ad);
        free(cq);
    }
    return overflow;
}

/*
 * Speculative verify, Gated DeltaNet form.  [blog] "The delta-rule wrinkle":
 * each token's corrected value u = beta (v - alpha S_{t-1} k) depends on the
 * state before it, so the T drafts' corrections come from a T x T
 * lower-triangular solve; [blog] "Speculative decoding": the checkpoint is
 * read against every draft, drafts become records behind the h committed
 * ones, a flush folds only the committed records.  Per tile, with committed
 * records (lam_j, u_j, k_j), j = 1..h, gamma over committed alphas and D over
 * draft alphas (D_{a:b} = prod_{l=a..b} alpha_l, 1 when empty):
 *   S_h x = gamma_{1:h} C x + sum_j gamma_{j+1:h} (k_j . x) u_j     (x = k_i, q_i)
 *   u_i + beta_i sum_{m<i} D_{m+1:i} (k_m . k_i) u_m = beta_i (v_i - D_{1:i} S_h k_i)
 *   o_i = D_{1:i} S_h q_i + sum_{m<=i} D_{m+1:i} (k_m . q_i) u_m
 * The system is solved by forward substitution, i = 1..T, one d_v-vector at
 * a time.  Then the committed records are folded on a flushing tile (as in
 * oc_spec_verify) and the drafts are stored as records (lam_i, u_i, k_i)
 * from slot (flush ? 0 : h).  rec_x holds u.
 */
int64_t oc_spec_verify_gdn(int64_t n, int dv, int dk, int cap, int T, double* C, double* rec_lam,
                           double* rec_x, double* rec_k, int32_t* h, const uint8_t* flush,
                           const double* q, const double* k, const double* v, const double* lam,
                           const double* beta, const uint8_t* active, double* out) {
    int64_t overflow = 0;
#pragma omp parallel reduction(+ : overflow)
    {
        double* ac = (double*)malloc(sizeof(double) * (size_t)(cap + 2));
        double* ad = (double*)malloc(sizeof(double) * (size_t)(T + 2));
        double* y = (double*)malloc(sizeof(double) * (size_t)dv);
        double* shk = (double*)malloc(sizeof(double) * (size_t)dv);
        double* shq = (double*)malloc(sizeof(double) * (size_t)dv);
        double* u = (double*)malloc(sizeof(double) * (size_t)T * dv); /* u[(i-1)*dv + r] */
#pragma omp for schedule(static)
        for (int64_t t = 0; t < n; ++t) {
            if (active && !active[t]) continue;
            const int ht = h[t];
            const int base = flush[t] ? 0 : ht;
            if (base + T > cap) { overflow += 1; continue; }
            double* Ct = C + t * (int64_t)dv * dk;
            double* lamt = rec_lam + t * (int64_t)cap;
            double* xt = rec_x + t * (int64_t)cap * dv;
            double* krt = rec_k + t * (int64_t)cap * dk;
            const double* qt = q + t * (int64_t)T * dk;
            const double* kt = k + t * (int64_t)T * dk;
            const double* vt = v + t * (int64_t)T * dv;
            const double* lt = lam + t * (int64_t)T;
            const double* bt = beta + t * (int64_t)T;
            double* ot = out + t * (int64_t)T * dv;
            for (int j = 1; j <= ht; ++j) ac[j] = exp(lamt[j - 1]);
            for (int i = 1; i <= T; ++i) ad[i] = exp(lt[i - 1]);
            const double gh = gamma_range(ac, 1, ht);
            for (int i = 1; i <= T; ++i) {
                const double* qi = qt + (int64_t)(i - 1) * dk;
                const double* ki = kt + (int64_t)(i - 1) * dk;
                /* the committed state S_h read at k_i and at q_i */
                matvec(Ct, ki, dv, dk, y);
                for (int r = 0; r < dv; ++r) shk[r] = gh * y[r];
                matvec(Ct, qi, dv, dk, y);
                for (int r = 0; r < dv; ++r) shq[r] = gh * y[r];
                for (int j = 1; j <= ht; ++j) {
                    const double g = gamma_range(ac, j + 1, ht);
                    const double* kj = krt + (int64_t)(j - 1) * dk;
                    const double wk = g * dot(kj, ki, dk), wq = g * dot(kj, qi, dk);
                    for (int r = 0; r < dv; ++r) {
                        shk[r] += wk * xt[(int64_t)(j - 1) * dv + r];
                        shq[r] += wq * xt[(int64_t)(j - 1) * dv + r];
                    }
                }
                /* row i of the triangular system, earlier drafts known */
                const double Di = gamma_range(ad, 1, i);
                double* ui = u + (int64_t)(i - 1) * dv;
                for (int r = 0; r < dv; ++r) ui[r] = bt[i - 1] * (vt[(int64_t)(i - 1) * dv + r] - Di * shk[r]);
                for (int m = 1; m < i; ++m) {
                    const double a = bt[i - 1] * gamma_range(ad, m + 1, i) * dot(kt + (int64_t)(m - 1) * dk, ki, dk);
                    for (int r = 0; r < dv; ++r) ui[r] -= a * u[(int64_t)(m - 1) * dv + r];
                }
                /* output of draft i */
                for (int r = 0; r < dv; ++r) ot[(int64_t)(i - 1) * dv + r] = Di * shq[r];
                for (int m = 1; m <= i; ++m) {
                    const double wgt = gamma_range(ad, m + 1, i) * dot(kt + (int64_t)(m - 1) * dk, qi, dk);
                    for (int r = 0; r < dv; ++r) ot[(int64_t)(i - 1) * dv + r] += wgt * u[(int64_t)(m - 1) * dv + r];
                }
            }
            if (flush[t]) {
                for (int r = 0; r < dv; ++r)
                    for (int c = 0; c < dk; ++c) {
                        double s = gh * Ct[(int64_t)r * dk + c];
                        for (int j = 1; j <= ht; ++j)
                            s += gamma_range(ac, j + 1, ht) * xt[(int64_t)(j - 1) * dv + r] * krt[(int64_t)(j - 1) * dk + c];
                        Ct[(int64_t)r * dk + c] = s;
                    }
                h[t] = 0;
            }
            for (int i = 0; i < T; ++i) {
                lamt[base + i] = lt[i];
                memcpy(xt + (int64_t)(base + i) * dv, u + (int64_t)i * dv, sizeof(double) * (size_t)dv);
                memcpy(krt + (int64_t)(base + i) * dk, kt + (int64_t)i * dk, sizeof(double) * (size_t)dk);
            }
        }
        free(ac);
        free(ad);
        free(y);
        free(shk);
        free(shq);
        free(u);
    }
    return overflow;
}

/*
 * Commit after a speculative verify ([blog]: "after sampling advances the
 * committed pointer by a"): h <- h + accepted for each selected tile.  The
 * verify step has already set h to 0 on a flushing tile.
 */
void oc_spec_commit(int64_t n, int32_t* h, const int32_t* accepted, const uint8_t* active) {
    for (int64_t t = 0; t < n; ++t)
        if (!active || active[t]) h[t] += accepted[t];
}

/*
 * Committed-pointer run of one row under speculative decoding with T drafts
 * per step and a ring of L committed records ([blog]: flush when h + T > L,
 * known before the step runs), simulated by counting what the ring holds:
 *   step s:  flush_s = (h + T > L) or forced_s;  emits (h, flush_s);
 *            then h = (flush_s ? 0 : h) + accepted_s.
 * forced may be NULL.
 */
void oc_spec_cursor_run(int L, int T, int32_t h0, int64_t n_steps, const int32_t* accepted,
                        const uint8_t* forced, int32_t* h_out, uint8_t* flush_out) {
    int32_t hc = h0;
    for (int64_t s = 0; s < n_steps; ++s) {
        int held = hc;          /* records the ring holds before the drafts */
        int room = L - held;    /* committed slots left */
        const int f = (room < T) || (forced && forced[s]);
        h_out[s] = hc;
        flush_out[s] = (uint8_t)f;
        hc = (f ? 0 : hc) + accepted[s];
    }
}
