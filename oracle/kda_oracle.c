/*
 * KDA oracle: plain, slow, token-by-token CPU reference in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP path.
 *
 * What it computes (Kimi Linear summary page, "The recurrent layers..."
 * paragraph: each step decays the state per channel, removes the old state's
 * projection onto the current key, then writes the new key/value pair; the
 * remio.ai page, section on how Kimi Linear uses its recurrent memory: KDA
 * extends Gated DeltaNet's delta rule with a finer, per-channel gate).  For
 * one head with a dk x dv state S whose rows are key channels:
 *
 *     S'  = Diag(exp(log_alpha_t)) S            decay each key channel
 *     u   = beta_t (v_t - S'^T k_t)             error of the old association
 *     S   = S' + k_t u^T                        delta-rule write
 *     o_t = S^T q_t                             read after the write
 *
 * Masked positions (Transformers issue report on Kimi Linear cached
 * continuation: padding must not advance the recurrent or convolution
 * state) leave S untouched and produce o_t = 0; their inputs are never read.
 *
 * Readings where the pages are silent: no 1/sqrt(dk) scale on q; o_t sees
 * token t's write; the optional L2 normalisation is x / sqrt(sum x^2 + 1e-6).
 *
 * Layouts (row-major): q,k,log_alpha [B,T,H,dk]; v,o [B,T,H,dv]; beta [B,T,H];
 * mask [B,T] (NULL = all valid); state [B,H,dk,dv].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define L2_EPS 1e-6

static void unit_copy(const double* x, double* y, int n, int normalise) {
    double s = 0.0;
    for (int i = 0; i < n; ++i) { y[i] = x[i]; s += x[i] * x[i]; }
    if (normalise) {
        double r = 1.0 / sqrt(s + L2_EPS);
        for (int i = 0; i < n; ++i) y[i] *= r;
    }
}

/* one valid token of the recurrence, in the order the summary page states */
static void kda_token(double* S, const double* q, const double* k, const double* v,
                      const double* log_alpha, double beta, double* o,
                      int dk, int dv, double* u) {
    for (int i = 0; i < dk; ++i) {                 /* decay: row i scaled by alpha_i */
        double a = exp(log_alpha[i]);
        double* row = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) row[j] *= a;
    }
    for (int j = 0; j < dv; ++j) {                 /* u = beta (v - S'^T k) */
        double p = 0.0;
        for (int i = 0; i < dk; ++i) p += S[(size_t)i * dv + j] * k[i];
        u[j] = beta * (v[j] - p);
    }
    for (int i = 0; i < dk; ++i) {                 /* S += k u^T */
        double* row = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) row[j] += k[i] * u[j];
    }
    for (int j = 0; j < dv; ++j) {                 /* o = S^T q */
        double s = 0.0;
        for (int i = 0; i < dk; ++i) s += S[(size_t)i * dv + j] * q[i];
        o[j] = s;
    }
}

/* Sequence of T tokens per (b,h).  init_state may be NULL (zeros).
 * Returns 0, or -1 on a bad argument / allocation failure. */
int kda_oracle_prefill(const double* q, const double* k, const double* v,
                       const double* log_alpha, const double* beta,
                       const uint8_t* mask, const double* init_state,
                       double* o, double* final_state,
                       int B, int T, int H, int dk, int dv, int l2norm_qk, int nthreads) {
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    int bad = 0;
    int nbh = B * H;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1) reduction(|:bad)
    for (int bh = 0; bh < nbh; ++bh) {
        int b = bh / H, h = bh % H;
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
        double* qn = (double*)malloc(sizeof(double) * (size_t)dk);
        double* kn = (double*)malloc(sizeof(double) * (size_t)dk);
        if (!S || !u || !qn || !kn) { bad = 1; free(S); free(u); free(qn); free(kn); continue; }
        size_t soff = ((size_t)b * H + h) * dk * dv;
        if (init_state) memcpy(S, init_state + soff, sizeof(double) * (size_t)dk * dv);
        else memset(S, 0, sizeof(double) * (size_t)dk * dv);
        for (int t = 0; t < T; ++t) {
            size_t row = ((size_t)b * T + t) * H + h;
            double* ot = o + row * dv;
            if (mask && !mask[(size_t)b * T + t]) {
                for (int j = 0; j < dv; ++j) ot[j] = 0.0;
                continue;
            }
            unit_copy(q + row * dk, qn, dk, l2norm_qk);
            unit_copy(k + row * dk, kn, dk, l2norm_qk);
            kda_token(S, qn, kn, v + row * dv, log_alpha + row * dk, beta[row], ot, dk, dv, u);
        }
        memcpy(final_state + soff, S, sizeof(double) * (size_t)dk * dv);
        free(S); free(u); free(qn); free(kn);
    }
    return bad ? -1 : 0;
}

/* One decode step per (b,h) on a state updated in place.  Layouts: q,k,log_alpha
 * [B,H,dk]; v,o [B,H,dv]; beta [B,H]; mask [B] (NULL = all valid). */
int kda_oracle_decode_step(const double* q, const double* k, const double* v,
                           const double* log_alpha, const double* beta, const uint8_t* mask,
                           double* state, double* o, int B, int H, int dk, int dv,
                           int l2norm_qk, int nthreads) {
    if (B < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    int bad = 0;
    int nbh = B * H;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1) reduction(|:bad)
    for (int bh = 0; bh < nbh; ++bh) {
        int b = bh / H;
        double* ot = o + (size_t)bh * dv;
        if (mask && !mask[b]) { for (int j = 0; j < dv; ++j) ot[j] = 0.0; continue; }
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
        double* qn = (double*)malloc(sizeof(double) * (size_t)dk);
        double* kn = (double*)malloc(sizeof(double) * (size_t)dk);
        if (!u || !qn || !kn) { bad = 1; free(u); free(qn); free(kn); continue; }
        unit_copy(q + (size_t)bh * dk, qn, dk, l2norm_qk);
        unit_copy(k + (size_t)bh * dk, kn, dk, l2norm_qk);
        kda_token(state + (size_t)bh * dk * dv, qn, kn, v + (size_t)bh * dv,
                  log_alpha + (size_t)bh * dk, beta[bh], ot, dk, dv, u);
        free(u); free(qn); free(kn);
    }
    return bad ? -1 : 0;
}

/* Depthwise causal short convolution with a cache, over the *compacted* sequence
 * (Transformers issue report on Kimi Linear: padded entries must not enter the
 * convolution window).  For each (b, channel c) the window history starts as the
 * W-1 cached inputs (oldest first; zeros if cache is NULL); each valid position
 * t computes y = bias + sum_j w[c,j] * window_j with window = (history, x_t),
 * then x_t joins the history.  Masked positions produce y = 0 and leave the
 * history alone.  The new cache is the final history.
 * Layouts: x,y [B,T,D]; w [D,W]; bias [D] or NULL; cache [B,W-1,D] or NULL;
 * new_cache [B,W-1,D] or NULL (not written). */
int kda_oracle_short_conv(const double* x, const double* w, const double* bias,
                          const uint8_t* mask, const double* cache, double* y, double* new_cache,
                          int B, int T, int D, int W, int silu) {
    if (B < 0 || T < 0 || D <= 0 || W <= 0 || W > 64) return -1;
    double hist[64];
    for (int b = 0; b < B; ++b) {
        for (int c = 0; c < D; ++c) {
            for (int j = 0; j < W - 1; ++j)
                hist[j] = cache ? cache[((size_t)b * (W - 1) + j) * D + c] : 0.0;
            for (int t = 0; t < T; ++t) {
                size_t idx = ((size_t)b * T + t) * D + c;
                if (mask && !mask[(size_t)b * T + t]) { y[idx] = 0.0; continue; }
                double xt = x[idx];
                double acc = bias ? bias[c] : 0.0;
                for (int j = 0; j < W - 1; ++j) acc += w[(size_t)c * W + j] * hist[j];
                acc += w[(size_t)c * W + (W - 1)] * xt;
                if (silu) acc = acc / (1.0 + exp(-acc));
                y[idx] = acc;
                for (int j = 0; j + 1 < W - 1; ++j) hist[j] = hist[j + 1];
                if (W > 1) hist[W - 2] = xt;
            }
            if (new_cache)
                for (int j = 0; j < W - 1; ++j) new_cache[((size_t)b * (W - 1) + j) * D + c] = hist[j];
        }
    }
    return 0;
}
