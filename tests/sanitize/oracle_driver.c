/*
 * The fp64 oracle (oracle/gdn_oracle.c) built with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py): every entry point on
 * small inputs, odd lengths and the argument errors, so that any out-of-bounds
 * access, leak or undefined operation in the oracle aborts the run.  The three
 * forms of the core recurrence must also agree here, as they do in the Python
 * pins.  Inputs come from a small linear congruential generator of this file
 * (the mixer's own arithmetic lives only in the oracle).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_core_sequential(int T, int dk, int dv, const double *q, const double *k, const double *v,
                           const double *g, const double *beta, double *S, double *o);
int oracle_core_chunked(int T, int dk, int dv, int C, const double *q, const double *k, const double *v,
                        const double *g, const double *beta, double *S, double *o);
int oracle_core_bruteforce(int T, int dk, int dv, const double *q, const double *k, const double *v,
                           const double *g, const double *beta, double *S, double *o);
void oracle_conv_silu_channel(int T, const double *x, const double *w4, const double *hist3, double *out);
void oracle_l2norm(int n, const double *x, double eps, double scale, double *out);
void oracle_gate_logits(int n, int Hv, const double *a, const double *b, const double *A_log,
                        const double *dt_bias, double *g, double *beta);
void oracle_gated_rmsnorm(int n, const double *o, const double *z, const double *w, double eps, double *y);
int oracle_prefill(int B, int T, int Hk, int Hv, int dk, int dv, int conv_width, int use_norm, double eps_l2,
                   double eps_norm, const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                   const float *beta, const uint16_t *z, const uint16_t *conv_w, const uint16_t *norm_w,
                   const float *state_in, const uint16_t *conv_state_in, int n_chains, const int32_t *chains,
                   double *y, double *state_out, uint16_t *conv_state_out, int n_threads);
int oracle_decode_step(int B, int Hk, int Hv, int dk, int dv, int conv_width, int use_norm, double eps_l2,
                       double eps_norm, const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                       const float *beta, const uint16_t *z, const uint16_t *conv_w, const uint16_t *norm_w,
                       const float *state, const uint16_t *conv_state, int n_chains, const int32_t *chains,
                       double *y, double *state_out, uint16_t *conv_state_out, int n_threads);

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double uni(void) { /* in [0, 1) */
    rng = rng * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng >> 11) * (1.0 / 9007199254740992.0);
}
static double sym(void) { return 2.0 * uni() - 1.0; }
static uint16_t bf16(double x) { /* truncation is enough for test data */
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}
static int failures = 0;
static void expect(int cond, const char *what) {
    if (!cond) {
        fprintf(stderr, "FAIL: %s\n", what);
        ++failures;
    }
}
static double maxdiff(const double *a, const double *b, size_t n) {
    double m = 0.0;
    for (size_t i = 0; i < n; ++i) m = fmax(m, fabs(a[i] - b[i]));
    return m;
}

static void core_forms(int T, int dk, int dv, int C) {
    double *q = malloc(sizeof(double) * T * dk), *k = malloc(sizeof(double) * T * dk);
    double *v = malloc(sizeof(double) * T * dv), *g = malloc(sizeof(double) * T), *be = malloc(sizeof(double) * T);
    double *S[3], *o[3];
    for (int t = 0; t < T; ++t) {
        double n = 0.0;
        for (int i = 0; i < dk; ++i) { k[t * dk + i] = sym(); n += k[t * dk + i] * k[t * dk + i]; }
        for (int i = 0; i < dk; ++i) { k[t * dk + i] /= sqrt(n); q[t * dk + i] = sym() / sqrt((double)dk); }
        for (int j = 0; j < dv; ++j) v[t * dv + j] = sym();
        g[t] = log(0.8 + 0.199 * uni());
        be[t] = uni();
    }
    for (int f = 0; f < 3; ++f) {
        S[f] = malloc(sizeof(double) * dk * dv);
        o[f] = malloc(sizeof(double) * T * dv);
        for (int i = 0; i < dk * dv; ++i) S[f][i] = 0.01 * (i % 7);
    }
    expect(oracle_core_sequential(T, dk, dv, q, k, v, g, be, S[0], o[0]) == 0, "sequential");
    expect(oracle_core_chunked(T, dk, dv, C, q, k, v, g, be, S[1], o[1]) == 0, "chunked");
    if (T <= 8) {
        expect(oracle_core_bruteforce(T, dk, dv, q, k, v, g, be, S[2], o[2]) == 0, "bruteforce");
        expect(maxdiff(o[0], o[2], (size_t)T * dv) < 1e-10 && maxdiff(S[0], S[2], (size_t)dk * dv) < 1e-10,
               "bruteforce agrees with sequential");
    }
    expect(maxdiff(o[0], o[1], (size_t)T * dv) < 1e-10 && maxdiff(S[0], S[1], (size_t)dk * dv) < 1e-10,
           "chunked agrees with sequential");
    expect(oracle_core_chunked(T, dk, dv, 0, q, k, v, g, be, S[1], o[1]) == -1, "chunk length 0 rejected");
    for (int f = 0; f < 3; ++f) { free(S[f]); free(o[f]); }
    free(q); free(k); free(v); free(g); free(be);
}

int main(void) {
    core_forms(7, 5, 3, 4);    /* ragged last chunk */
    core_forms(8, 8, 8, 8);
    core_forms(33, 16, 12, 8);

    /* elementwise pieces */
    double x[9], w4[4] = {0.3, -0.2, 0.5, 1.0}, hist[3] = {0.1, -0.4, 0.2}, out[9], y[9], z[9], wn[9];
    for (int i = 0; i < 9; ++i) { x[i] = sym(); z[i] = sym(); wn[i] = 1.0 + 0.02 * sym(); }
    oracle_conv_silu_channel(9, x, w4, hist, out);
    oracle_conv_silu_channel(9, x, w4, NULL, out);
    oracle_l2norm(9, x, 1e-6, 1.0, out);
    oracle_gated_rmsnorm(9, x, z, wn, 1e-6, y);
    double a[6], bb[6], Al[3] = {0.1, 1.0, 2.7}, dt[3] = {-4.0, -3.0, -2.5}, gg[6], bt[6];
    for (int i = 0; i < 6; ++i) { a[i] = 3.0 * sym(); bb[i] = 3.0 * sym(); }
    oracle_gate_logits(2, 3, a, bb, Al, dt, gg, bt);
    for (int i = 0; i < 6; ++i) expect(gg[i] < 0.0 && bt[i] > 0.0 && bt[i] < 1.0, "gate logits ranges");

    /* the whole layer, small head widths, two sequences, conv + norm, a chain subset */
    const int B = 2, T = 70, Hk = 2, Hv = 4, dk = 16, dv = 16;
    const size_t Cc = (size_t)2 * Hk * dk + (size_t)Hv * dv;
    uint16_t *q = malloc(2 * B * T * Hk * dk), *k = malloc(2 * B * T * Hk * dk), *v = malloc(2 * B * T * Hv * dv);
    uint16_t *zz = malloc(2 * B * T * Hv * dv), *cw = malloc(2 * Cc * 4), *nw = malloc(2 * dv);
    uint16_t *cs_in = malloc(2 * B * 3 * Cc), *cs_out = malloc(2 * B * 3 * Cc);
    float *g = malloc(4 * B * T * Hv), *be = malloc(4 * B * T * Hv), *st = malloc(4 * B * Hv * dk * dv);
    for (int i = 0; i < B * T * Hk * dk; ++i) { q[i] = bf16(sym()); k[i] = bf16(sym()); }
    for (int i = 0; i < B * T * Hv * dv; ++i) { v[i] = bf16(sym()); zz[i] = bf16(sym()); }
    for (size_t i = 0; i < Cc * 4; ++i) cw[i] = bf16(0.5 * sym());
    for (int i = 0; i < dv; ++i) nw[i] = bf16(1.0 + 0.02 * sym());
    for (size_t i = 0; i < B * 3 * Cc; ++i) cs_in[i] = bf16(sym());
    for (int i = 0; i < B * T * Hv; ++i) { g[i] = (float)log(0.8 + 0.199 * uni()); be[i] = (float)uni(); }
    for (int i = 0; i < B * Hv * dk * dv; ++i) st[i] = (float)(0.1 * sym());
    const int32_t chains[3] = {0, 5, 7};
    double *yy = malloc(sizeof(double) * B * Hv * T * dv), *so = malloc(sizeof(double) * B * Hv * dk * dv);
    expect(oracle_prefill(B, T, Hk, Hv, dk, dv, 4, 1, 1e-6, 1e-6, q, k, v, g, be, zz, cw, nw, st, cs_in, 0, NULL, yy,
                          so, cs_out, 1) == 0, "prefill, all chains");
    expect(oracle_prefill(B, T, Hk, Hv, dk, dv, 4, 1, 1e-6, 1e-6, q, k, v, g, be, zz, cw, nw, NULL, NULL, 3, chains,
                          yy, so, NULL, 1) == 0, "prefill, chain subset, zero states");
    expect(oracle_prefill(B, T, Hk, Hv, dk, dv, 0, 0, 1e-6, 1e-6, q, k, v, g, be, NULL, NULL, NULL, NULL, NULL, 0,
                          NULL, yy, so, NULL, 1) == 0, "prefill, raw path");
    expect(oracle_decode_step(B, Hk, Hv, dk, dv, 4, 1, 1e-6, 1e-6, q, k, v, g, be, zz, cw, nw, st, cs_in, 0, NULL, yy,
                              so, cs_out, 1) == 0, "decode step");
    /* argument errors */
    expect(oracle_prefill(B, T, Hk, 3, dk, dv, 4, 1, 1e-6, 1e-6, q, k, v, g, be, zz, cw, nw, st, cs_in, 0, NULL, yy,
                          so, cs_out, 1) == -1, "Hv not a multiple of Hk");
    expect(oracle_prefill(B, T, Hk, Hv, dk, dv, 3, 1, 1e-6, 1e-6, q, k, v, g, be, zz, cw, nw, st, cs_in, 0, NULL, yy,
                          so, cs_out, 1) == -1, "conv width 3");
    expect(oracle_prefill(B, T, Hk, Hv, dk, dv, 4, 1, 1e-6, 1e-6, q, k, v, g, be, NULL, cw, nw, st, cs_in, 0, NULL, yy,
                          so, cs_out, 1) == -1, "norm without z");
    expect(oracle_prefill(0, T, Hk, Hv, dk, dv, 4, 1, 1e-6, 1e-6, q, k, v, g, be, zz, cw, nw, st, cs_in, 0, NULL, yy,
                          so, cs_out, 1) == -1, "B = 0");
    free(q); free(k); free(v); free(zz); free(cw); free(nw); free(cs_in); free(cs_out);
    free(g); free(be); free(st); free(yy); free(so);
    if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
    else printf("oracle under sanitizers: all passed\n");
    return failures ? 1 : 0;
}
