/*
 * gdn_oracle.c -- plain CPU oracle for the gated delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library never
 * links, loads or calls it, and the two share no source.
 *
 * What it computes, in double precision, one token at a time, with no chunking:
 *
 *   Source: "Qwen3.8-27B 架构深读: Gated DeltaNet 混合线性注意力与 262K 长上下文"
 *   (feifeigd.github.io blog, 2026-08-17), section 三 (Gated DeltaNet), the
 *   gated delta-rule equation
 *
 *       S_t = g_t S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T.
 *
 *   Per head, S is a d_v x d_k matrix.  The equation is evaluated as written,
 *   for each token t: the prediction error of the previous state,
 *
 *       u_t = v_t - S_{t-1} k_t,
 *
 *   then the new state S_t = g_t S_{t-1} + beta_t u_t k_t^T, then the read-out
 *   o_t = S_t q_t.
 *
 *   Readings taken where the page is loose:
 *   - Orientation.  In the equation the correction is (v - S k) k^T, so S maps
 *     keys (length d_k) to values (length d_v): S is d_v x d_k.
 *   - The error term reads S_{t-1}, the state before the gate is applied, so
 *     the transition applied to S from the right is g_t I - beta_t k_t k_t^T.
 *   - Output.  The page gives no GDN read-out; the linear-attention formula in
 *     the same section reads the memory with the query.  Here o_t = S_t q_t,
 *     identity feature map, no 1/sqrt(d) scale.
 *   - Gate and strength are one scalar each per (token, head); the page decays
 *     the whole matrix by the token's gate.
 *   - Sequences in a packed batch never share state: each starts from its own
 *     initial state (zeros when none is given).  A sequence of length zero
 *     returns its initial state unchanged.
 *
 *   Variants (gdn_oracle_run_variant), from the same section's equations:
 *   - bit 1, no gate: g_t = 1, the plain delta rule S_t = S_{t-1} +
 *     beta_t (v_t - S_{t-1} k_t) k_t^T (g is ignored and may be NULL);
 *   - bit 2, no erase: the recall term is dropped, S_t = g_t S_{t-1} +
 *     beta_t v_t k_t^T, the linear-attention write (with both bits and
 *     beta = 1: S_t = S_{t-1} + v_t k_t^T, plain linear attention).
 *
 * Arithmetic: plain loops, j ascending, no fused multiply-add contraction
 * (built with -O2 -fno-fast-math -ffp-contract=off).  Because each token's
 * arithmetic depends only on the state and that token, splitting a sequence
 * into segments and carrying the state gives bit-identical results.
 *
 * Layouts (all row-major, contiguous):
 *   q, k     [N][H][dk]        v [N][H][dv]        g, beta [N][H]
 *   o        [N][H][dv]
 *   s_init   [n_seq][H][dv][dk]   (NULL: zeros)
 *   s_final  [n_seq][H][dv][dk]   (may alias s_init)
 *   cu_seqlens [n_seq+1], non-decreasing, cu[0] = 0, cu[n_seq] = N
 *   (NULL: one sequence holding all N tokens; n_seq must then be 1).
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v, *g, *beta, *s_init;
    const int64_t *cu;
    double *o, *s_final;
    int64_t n_seq, H, dk, dv;
    int variant;       /* bit 1: no gate; bit 2: no erase term */
    int64_t next_unit; /* shared work counter, advanced atomically */
} gdn_oracle_job;

static void run_unit(const gdn_oracle_job *J, int64_t unit, double *r) {
    const int64_t H = J->H, dk = J->dk, dv = J->dv;
    const int64_t s = unit / H, h = unit % H;
    double *S = J->s_final + (s * H + h) * dv * dk;
    if (J->s_init) {
        const double *S0 = J->s_init + (s * H + h) * dv * dk;
        if (S0 != S) memcpy(S, S0, (size_t)(dv * dk) * sizeof(double));
    } else {
        memset(S, 0, (size_t)(dv * dk) * sizeof(double));
    }
    const int64_t t0 = J->cu ? J->cu[s] : 0;
    const int64_t t1 = J->cu ? J->cu[s + 1] : t0;
    for (int64_t t = t0; t < t1; ++t) {
        const double *kt = J->k + (t * H + h) * dk;
        const double *qt = J->q + (t * H + h) * dk;
        const double *vt = J->v + (t * H + h) * dv;
        const double gt = (J->variant & 1) ? 1.0 : J->g[t * H + h];
        const double bt = J->beta[t * H + h];
        double *ot = J->o + (t * H + h) * dv;
        /* S_{t-1} k_t, the part of the error term read from the previous state
           (absent without the erase term) */
        for (int64_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            if (!(J->variant & 2))
                for (int64_t j = 0; j < dk; ++j) acc += S[i * dk + j] * kt[j];
            r[i] = acc;
        }
        /* S_t = g_t S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T */
        for (int64_t i = 0; i < dv; ++i) {
            const double c = bt * (vt[i] - r[i]);
            for (int64_t j = 0; j < dk; ++j) S[i * dk + j] = gt * S[i * dk + j] + c * kt[j];
        }
        /* o_t = S_t q_t */
        for (int64_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < dk; ++j) acc += S[i * dk + j] * qt[j];
            ot[i] = acc;
        }
    }
}

static void *worker(void *arg) {
    gdn_oracle_job *J = (gdn_oracle_job *)arg;
    double *r = (double *)malloc((size_t)J->dv * sizeof(double));
    if (!r) return (void *)1;
    const int64_t n_units = J->n_seq * J->H;
    for (;;) {
        const int64_t u = __atomic_fetch_add(&J->next_unit, 1, __ATOMIC_RELAXED);
        if (u >= n_units) break;
        run_unit(J, u, r);
    }
    free(r);
    return NULL;
}

/* Returns 0 on success, a negative code on invalid arguments (nothing is
 * written then), or -100 when a thread or buffer could not be created. */
int gdn_oracle_run_variant(const double *q, const double *k, const double *v,
                           const double *g, const double *beta,
                           const int64_t *cu_seqlens, int64_t n_seq, int64_t total_tokens,
                           int64_t H, int64_t dk, int64_t dv,
                           const double *s_init, double *o, double *s_final, int n_threads, int variant) {
    if (n_seq < 0 || total_tokens < 0 || H <= 0 || dk <= 0 || dv <= 0 || (variant & ~3)) return -1;
    if (!s_final) return -2;
    if (total_tokens > 0 && (!q || !k || !v || (!g && !(variant & 1)) || !beta || !o)) return -2;
    if (!cu_seqlens) {
        if (n_seq != 1) return -3;
    } else {
        if (cu_seqlens[0] != 0 || cu_seqlens[n_seq] != total_tokens) return -3;
        for (int64_t s = 0; s < n_seq; ++s)
            if (cu_seqlens[s + 1] < cu_seqlens[s]) return -3;
    }
    int64_t one_seq[2] = {0, total_tokens};
    gdn_oracle_job J;
    J.q = q; J.k = k; J.v = v; J.g = g; J.beta = beta; J.s_init = s_init;
    J.cu = cu_seqlens ? cu_seqlens : one_seq;
    J.o = o; J.s_final = s_final;
    J.n_seq = n_seq; J.H = H; J.dk = dk; J.dv = dv;
    J.variant = variant;
    J.next_unit = 0;
    if (n_seq == 0) return 0;

    if (n_threads < 1) n_threads = 1;
    if ((int64_t)n_threads > n_seq * H) n_threads = (int)(n_seq * H);
    pthread_t *tid = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!tid) return -100;
    int started = 0, failed = 0;
    for (int i = 1; i < n_threads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, &J) != 0) { failed = 1; break; }
        ++started;
    }
    if (worker(&J) != NULL) failed = 1;
    for (int i = 1; i <= started; ++i) {
        void *ret = NULL;
        pthread_join(tid[i], &ret);
        if (ret != NULL) failed = 1;
    }
    free(tid);
    return failed ? -100 : 0;
}

/* The gated delta rule itself (variant 0). */
int gdn_oracle_run(const double *q, const double *k, const double *v,
                   const double *g, const double *beta,
                   const int64_t *cu_seqlens, int64_t n_seq, int64_t total_tokens,
                   int64_t H, int64_t dk, int64_t dv,
                   const double *s_init, double *o, double *s_final, int n_threads) {
    return gdn_oracle_run_variant(q, k, v, g, beta, cu_seqlens, n_seq, total_tokens, H, dk, dv, s_init, o, s_final,
                                  n_threads, 0);
}
