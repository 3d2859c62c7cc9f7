/*
 * kda_oracle.c -- plain, slow, fp64 CPU reference of the KDA gated delta rule.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline may load this file's library. It shares no code, header, table or
 * helper with the GPU library, and the GPU library never calls it.
 *
 * What it computes, per (sequence, head), token by token, for t = 1..T:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T (scale * q_t),        alpha_t = exp(log_alpha_t)  (per key channel)
 *
 * S is d_k x d_v, row i = key channel i, so Diag(alpha) scales rows. This is the
 * KDA update as written at the end of the "ten questions" page
 * (jokeuncle.github.io, Kimi K3 KDA math for beginners: the closing
 * symbol-by-symbol reading, with the 2x2 memory of Q3-Q8). The loop below takes
 * the step in the order the bra-ket derivation page (mynewscn.com, opening KDA
 * state-update equations) gives it, transposed to the d_k x d_v orientation:
 *
 *     forget:   S~ = Diag(alpha_t) S_{t-1}
 *     recall:   v^ = S~^T k_t                      (what the key reads now)
 *     error:    e  = beta_t (v_t - v^)
 *     write:    S_t = S~ + k_t e^T
 *     read out: o_t = S_t^T (scale q_t)            (scale = d_k^{-1/2} on that page)
 *
 * Expanding "write" with "error" gives the formula above exactly, so no
 * reordering is involved. With delta_rule == 0 the recall/error pair is
 * dropped (e = beta_t v_t): S_t = Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T, the
 * gated linear attention of the GPT-2 -> Kimi K3 essay
 * (yichencityu.github.io, section 8), and with alpha = beta = 1 the plain
 * linear attention of the bra-ket page, section 1.1.
 *
 * Sequences are packed along the token axis: sequence s owns tokens
 * [cu_seqlens[s], cu_seqlens[s+1]). Every (sequence, head) pair is independent;
 * pthreads split the pairs, never the token loop.
 *
 * Pinned by tests/test_oracle_pins.py (worked examples, closed forms, brute
 * force, invariants).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t n_seqs;
    const int64_t *cu_seqlens;
    int H, dk, dv;
    const double *q, *k, *v, *log_alpha, *beta;
    double scale;
    int delta_rule;
    const double *h0;
    double *o, *hT;
    int n_threads;
    int thread_id;
    int failed;
} oracle_job;

/* One (sequence, head) pair, token by token. Returns 0 on success. */
static int run_pair(const oracle_job *J, int64_t s, int h)
{
    const int H = J->H, dk = J->dk, dv = J->dv;
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *vhat = (double *)malloc(sizeof(double) * (size_t)dv);
    double *e = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!S || !vhat || !e) {
        free(S); free(vhat); free(e);
        return 1;
    }
    if (J->h0) {
        memcpy(S, J->h0 + ((size_t)s * H + h) * dk * dv, sizeof(double) * (size_t)dk * dv);
    } else {
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
    }

    for (int64_t t = J->cu_seqlens[s]; t < J->cu_seqlens[s + 1]; ++t) {
        const double *qt = J->q + ((size_t)t * H + h) * dk;
        const double *kt = J->k + ((size_t)t * H + h) * dk;
        const double *vt = J->v + ((size_t)t * H + h) * dv;
        const double *lat = J->log_alpha + ((size_t)t * H + h) * dk;
        const double bt = J->beta[(size_t)t * H + h];

        /* forget: S~ = Diag(alpha_t) S_{t-1}, row i scaled by alpha_t[i] */
        for (int i = 0; i < dk; ++i) {
            const double a = exp(lat[i]);
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
        }

        /* recall and error: v^ = S~^T k_t, e = beta_t (v_t - v^) */
        if (J->delta_rule) {
            for (int j = 0; j < dv; ++j) vhat[j] = 0.0;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) vhat[j] += S[(size_t)i * dv + j] * kt[i];
            for (int j = 0; j < dv; ++j) e[j] = bt * (vt[j] - vhat[j]);
        } else {
            for (int j = 0; j < dv; ++j) e[j] = bt * vt[j];
        }

        /* write: S_t = S~ + k_t e^T */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += kt[i] * e[j];

        /* read out after the write: o_t = S_t^T (scale q_t) */
        double *ot = J->o + ((size_t)t * H + h) * dv;
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * (J->scale * qt[i]);
            ot[j] = acc;
        }
    }

    if (J->hT) memcpy(J->hT + ((size_t)s * H + h) * dk * dv, S, sizeof(double) * (size_t)dk * dv);
    free(S); free(vhat); free(e);
    return 0;
}

static void *worker(void *arg)
{
    oracle_job *J = (oracle_job *)arg;
    const int64_t n_pairs = J->n_seqs * J->H;
    for (int64_t p = J->thread_id; p < n_pairs; p += J->n_threads) {
        if (run_pair(J, p / J->H, (int)(p % J->H))) J->failed = 1;
    }
    return NULL;
}

/*
 * kda_oracle_fwd -- fp64 reference over packed sequences.
 *   q, k        [T_total, H, dk]     v, o [T_total, H, dv]
 *   log_alpha   [T_total, H, dk]     beta [T_total, H]
 *   h0, hT      [n_seqs, H, dk, dv]  (h0 NULL = zero state, hT NULL = not returned)
 *   cu_seqlens  [n_seqs + 1], non-decreasing, cu_seqlens[0] == 0
 * Returns 0 on success, 1 on bad arguments, 2 on allocation or thread failure.
 */
int kda_oracle_fwd(int64_t n_seqs, const int64_t *cu_seqlens, int H, int dk, int dv,
                   const double *q, const double *k, const double *v,
                   const double *log_alpha, const double *beta, double scale, int delta_rule,
                   const double *h0, double *o, double *hT, int n_threads)
{
    if (n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || !cu_seqlens) return 1;
    if (n_seqs > 0 && cu_seqlens[0] != 0) return 1;
    for (int64_t s = 0; s < n_seqs; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s]) return 1;
    if (n_seqs > 0 && cu_seqlens[n_seqs] > 0 && (!q || !k || !v || !log_alpha || !beta || !o))
        return 1;
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;

    oracle_job jobs[256];
    pthread_t tids[256];
    int started = 0, failed = 0;
    for (int w = 0; w < n_threads; ++w) {
        jobs[w] = (oracle_job){n_seqs, cu_seqlens, H, dk, dv, q, k, v, log_alpha, beta, scale,
                               delta_rule, h0, o, hT, n_threads, w, 0};
    }
    for (int w = 1; w < n_threads; ++w) {
        if (pthread_create(&tids[w], NULL, worker, &jobs[w]) != 0) {
            failed = 1;
            break;
        }
        started = w;
    }
    if (!failed) worker(&jobs[0]);
    for (int w = 1; w <= started; ++w) pthread_join(tids[w], NULL);
    if (failed) return 2;
    for (int w = 0; w < n_threads; ++w)
        if (jobs[w].failed) return 2;
    return 0;
}
