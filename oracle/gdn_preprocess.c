/*
 * gdn_preprocess.c -- plain CPU oracle for the pre-processing in front of the
 * gated delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library never
 * links, loads or calls it, and the two share no source.
 *
 * What the pages fix:
 *   - "Layouts híbridos: três DeltaNet, uma attention" (llmdeepdive.com),
 *     section Conceito: the DeltaNet layers carry a convolution of kernel 4
 *     next to their gated state.
 *   - "Qwen3.8-27B 架构深读" (feifeigd.github.io, 2026-08-17), section 三:
 *     one gate g and one write strength beta per token, g deciding how much
 *     to forget (the page leaves normalisation details out).
 * Readings taken where the pages are silent (the same on the GPU):
 *   - The convolution is causal and depthwise (one 4-tap filter per channel)
 *     over the tokens of each sequence, applied to q, k and v.  Tap 3
 *     multiplies the current token, tap 0 the token three back.  Before a
 *     sequence's first token the window holds the sequence's conv state: the
 *     last three raw inputs of its previous part (zeros when none is given).
 *   - Activation after the convolution: none by default (the pages name
 *     none); SiLU, y * sigmoid(y), on request.
 *   - q and k are then L2-normalised per (token, head) over their d
 *     channels (a zero vector stays zero); v is not.
 *   - beta = sigmoid(b) and g = exp(-softplus(a + bias_h)) from per-(token,
 *     head) logits a, b and an optional per-head bias.
 *   - The conv state returned for each sequence holds its last three raw
 *     inputs (for a sequence shorter than three, shifted in from the state it
 *     started with), so a sequence processed in parts, each part's returned
 *     state fed to the next, gives the one-shot result exactly.
 *
 * Layouts (row-major, contiguous):
 *   xq, xk, xv, yq, yk, yv   [N][H][d]
 *   w                         [3][H][d][4]   (tensor q, k, v; head; channel; tap)
 *   state_in, state_out       [n_seq][3][3][H][d]   (tensor; tap 0..2 = tokens
 *                             three, two and one before the part; head; channel)
 *   a_logit, b_logit, g, beta [N][H];   bias [H] or NULL
 *   cu_seqlens [n_seq + 1] (NULL: one sequence of N tokens; n_seq must be 1)
 * Plain loops in double precision (-O2 -fno-fast-math -ffp-contract=off).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static double softplus(double x) { return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

/* raw input of tensor tau, token p (< t0 reads the part's starting state) */
static double raw(const double *const x[3], const double *state_in, int64_t s, int tau, int64_t p, int64_t t0,
                  int64_t H, int64_t d, int64_t h, int64_t c) {
    if (p >= t0) return x[tau][(p * H + h) * d + c];
    if (!state_in) return 0.0;
    const int64_t i = 3 - (t0 - p); /* 0..2 */
    return state_in[(((s * 3 + tau) * 3 + i) * H + h) * d + c];
}

int gdn_oracle_preprocess(const double *xq, const double *xk, const double *xv, const double *w,
                          const double *state_in, const double *a_logit, const double *b_logit, const double *bias,
                          const int64_t *cu_seqlens, int64_t n_seq, int64_t N, int64_t H, int64_t d, int activation,
                          double *yq, double *yk, double *yv, double *g, double *beta, double *state_out) {
    if (n_seq < 0 || N < 0 || H <= 0 || d <= 0 || (activation != 0 && activation != 1)) return -1;
    if (N > 0 && (!xq || !xk || !xv || !w || !a_logit || !b_logit || !yq || !yk || !yv || !g || !beta)) return -2;
    if (n_seq > 0 && !state_out) return -2;
    if (!cu_seqlens) {
        if (n_seq != 1) return -3;
    } else {
        if (cu_seqlens[0] != 0 || cu_seqlens[n_seq] != N) return -3;
        for (int64_t s = 0; s < n_seq; ++s)
            if (cu_seqlens[s + 1] < cu_seqlens[s]) return -3;
    }
    const double *const x[3] = {xq, xk, xv};
    double *const y[3] = {yq, yk, yv};
    double *buf = (double *)malloc((size_t)d * sizeof(double));
    if (!buf) return -100;

    for (int64_t s = 0; s < n_seq; ++s) {
        const int64_t t0 = cu_seqlens ? cu_seqlens[s] : 0;
        const int64_t t1 = cu_seqlens ? cu_seqlens[s + 1] : N;
        for (int64_t t = t0; t < t1; ++t) {
            for (int64_t h = 0; h < H; ++h) {
                for (int tau = 0; tau < 3; ++tau) {
                    for (int64_t c = 0; c < d; ++c) {
                        double acc = 0.0;
                        for (int j = 0; j < 4; ++j)
                            acc += w[((tau * H + h) * d + c) * 4 + j] * raw(x, state_in, s, tau, t - 3 + j, t0, H, d, h, c);
                        buf[c] = activation ? acc * sigmoid(acc) : acc;
                    }
                    double scale = 1.0;
                    if (tau < 2) {
                        double ss = 0.0;
                        for (int64_t c = 0; c < d; ++c) ss += buf[c] * buf[c];
                        if (ss > 0.0) scale = 1.0 / sqrt(ss);
                    }
                    for (int64_t c = 0; c < d; ++c) y[tau][(t * H + h) * d + c] = buf[c] * scale;
                }
                const double bh = bias ? bias[h] : 0.0;
                beta[t * H + h] = sigmoid(b_logit[t * H + h]);
                g[t * H + h] = exp(-softplus(a_logit[t * H + h] + bh));
            }
        }
        /* the last three raw inputs (read before any of them is written, so
           state_out may alias state_in) */
        const int64_t per = 3 * 3 * H * d;
        double *tmp = (double *)malloc((size_t)per * sizeof(double));
        if (!tmp) {
            free(buf);
            return -100;
        }
        for (int tau = 0; tau < 3; ++tau)
            for (int i = 0; i < 3; ++i)
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t c = 0; c < d; ++c)
                        tmp[((tau * 3 + i) * H + h) * d + c] = raw(x, state_in, s, tau, t1 - 3 + i, t0, H, d, h, c);
        for (int64_t e = 0; e < per; ++e) state_out[s * per + e] = tmp[e];
        free(tmp);
    }
    free(buf);
    return 0;
}
