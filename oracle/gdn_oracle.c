/*
 * gdn_oracle.c -- plain, slow fp64 CPU oracle of the Gated DeltaNet mixer hot
 * path (causal conv + SiLU, q/k L2 normalisation, gated delta rule, gated
 * RMSNorm).
 *
 * TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the bench's
 * CPU-baseline leg are the only callers.  The mixer library never calls,
 * links or includes anything from here, and this file includes nothing from
 * the library: the two share no code, header, table or constant.
 *
 * Every input is widened exactly (bf16 bits or fp32 -> fp64); all arithmetic
 * is fp64 with libm exp/sqrt.  Sources, cited by page title and section:
 *
 *  [HQ]  "How Qwen3.5 works" (azmle112.github.io qwen35-technical-analysis):
 *        §9.3 causal depthwise conv + SiLU on q/k/v only; §9.4 q/k L2
 *        normalisation with eps inside the root and the 1/sqrt(d_k) query
 *        scale, heads expanded by repeat_interleave; §9.6 the recurrence in
 *        the order decay -> predict -> correct -> read, state S in R^{dk x dv};
 *        §9.8 the 2x2 worked example; §9.9 RMSNormGated; §9.11 the chunked
 *        (unit lower-triangular) form; §13.1/§13.3 conv and recurrent state.
 *  [FE]  "Qwen3.8-27B" model spec (docs.theformalera.com), compute-graph nodes
 *        table: gdn.conv  y[t,c] = silu(sum_{j<4} w[c,j] x[t+j-3,c]);
 *        gdn.core (qk_l2norm_eps = 1e-6, q scaled by 1/sqrt(128), value head
 *        h reads key head h/ratio); gdn.norm  y = w * x/sqrt(mean(x^2)+eps) *
 *        silu(z), eps = 1e-6.
 *  [AD]  Qwen3.5-4B architecture page (ayushdeva.com), delta-rule derivation
 *        and the d = 2 single-head walkthrough.
 *  [HQ]  §9.5 the gates from their logits: beta = sigmoid(b),
 *        g = -exp(A_log) softplus(a + dt_bias), alpha = exp(g).
 *
 * Memory orientation: the state is stored K-major, S[i][j] with i a key
 * dimension and j a value dimension ([HQ] §9.1 orientation S in R^{dk x dv},
 * read-out o = S^T q).  The [FE] formula writes the transposed matrix
 * (S in R^{dv x dk}, o = S q); the two are the same operation.
 *
 * Parity pins live in tests/test_oracle_pins.py; every function below has at
 * least one pin that does not go through this file's own arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double silu(double x) { return x / (1.0 + exp(-x)); }

/* ------------------------------------------------------------------------ */
/* Building blocks                                                           */
/* ------------------------------------------------------------------------ */

/*
 * Causal depthwise conv + SiLU of ONE channel over T steps ([FE] gdn.conv,
 * [HQ] §9.3): u[t] = silu(sum_{j=0..3} w[j] * x[t+j-3]).  w[3] multiplies the
 * current step and w[0] the step three back.  Steps before t = 0 come from
 * hist[0..2] (hist[s] is step s-3, oldest first) or are zero when hist is NULL.
 */
void oracle_conv_silu_channel(int T, const double *x, const double *w4,
                              const double *hist3, double *u)
{
    for (int t = 0; t < T; ++t) {
        double acc = 0.0;
        for (int j = 0; j < 4; ++j) {
            int tau = t + j - 3;
            double xv;
            if (tau >= 0)
                xv = x[tau];
            else
                xv = hist3 ? hist3[3 + tau] : 0.0;
            acc += w4[j] * xv;
        }
        u[t] = silu(acc);
    }
}

/* L2 normalisation with eps inside the root, then a scale ([HQ] §9.4):
 * out = scale * x / sqrt(sum x^2 + eps). */
void oracle_l2norm(int n, const double *x, double eps, double scale, double *out)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i)
        ss += x[i] * x[i];
    double inv = scale / sqrt(ss + eps);
    for (int i = 0; i < n; ++i)
        out[i] = x[i] * inv;
}

/*
 * The gates from their logits, [HQ] §9.5: for n tokens of Hv value heads (a, b
 * laid out [n][Hv], A_log and dt_bias per head),
 *   beta = sigmoid(b) = 1 / (1 + e^{-b}),
 *   g    = -exp(A_log[h]) * softplus(a + dt_bias[h]),  softplus(x) = ln(1 + e^x)
 * (ln(1 + e^x) evaluated as x + ln(1 + e^{-x}) for x > 0 so e^x cannot overflow).
 */
void oracle_gate_logits(int n, int Hv, const double *a, const double *b, const double *A_log,
                        const double *dt_bias, double *g, double *beta)
{
    for (int t = 0; t < n; ++t)
        for (int h = 0; h < Hv; ++h) {
            const double x = a[(size_t)t * Hv + h] + dt_bias[h];
            const double sp = x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
            g[(size_t)t * Hv + h] = -exp(A_log[h]) * sp;
            beta[(size_t)t * Hv + h] = 1.0 / (1.0 + exp(-b[(size_t)t * Hv + h]));
        }
}

/* Gated RMSNorm of one head vector ([FE] gdn.norm, [HQ] §9.9):
 * y = w * o / sqrt(mean(o^2) + eps) * silu(z).  Plain w (not 1 + w). */
void oracle_gated_rmsnorm(int n, const double *o, const double *z, const double *w,
                          double eps, double *y)
{
    double ms = 0.0;
    for (int i = 0; i < n; ++i)
        ms += o[i] * o[i];
    ms /= (double)n;
    double inv = 1.0 / sqrt(ms + eps);
    for (int i = 0; i < n; ++i)
        y[i] = w[i] * (o[i] * inv) * silu(z[i]);
}

/*
 * One token of the gated delta rule on a K-major state S[dk][dv] ([HQ] §9.6):
 *   decay    S <- exp(g) S
 *   predict  p = S^T k
 *   correct  d = beta (v - p);  S <- S + k d^T
 *   read     o = S^T q
 * p and d are caller scratch of length dv.
 */
static void core_step(int dk, int dv, double *S, const double *q, const double *k,
                      const double *v, double g, double beta, double *o,
                      double *p, double *d)
{
    double a = exp(g);
    for (int i = 0; i < dk * dv; ++i)
        S[i] *= a;
    for (int j = 0; j < dv; ++j)
        p[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            p[j] += S[i * dv + j] * k[i];
    for (int j = 0; j < dv; ++j)
        d[j] = beta * (v[j] - p[j]);
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[i * dv + j] += k[i] * d[j];
    for (int j = 0; j < dv; ++j)
        o[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            o[j] += S[i * dv + j] * q[i];
}

/*
 * Core recurrence, token by token ([HQ] §9.6), on already-normalised keys and
 * already-scaled queries.  q,k [T][dk]; v [T][dv]; g, beta [T];
 * S [dk][dv] in/out; o [T][dv].  Returns 0, or -1 if scratch allocation fails.
 */
int oracle_core_sequential(int T, int dk, int dv, const double *q, const double *k,
                           const double *v, const double *g, const double *beta,
                           double *S, double *o)
{
    double *p = malloc(sizeof(double) * (size_t)dv * 2);
    if (!p)
        return -1;
    for (int t = 0; t < T; ++t)
        core_step(dk, dv, S, q + (size_t)t * dk, k + (size_t)t * dk, v + (size_t)t * dv,
                  g[t], beta[t], o + (size_t)t * dv, p, p + dv);
    free(p);
    return 0;
}

/*
 * Chunked form of the same recurrence ([HQ] §9.11), used only to cross-check
 * oracle_core_sequential.  Per chunk of n <= C tokens with start state S0:
 *   G_i = sum_{s<=i} g_s (cumulative log-decay inside the chunk),
 *   R_ij = exp(G_i - G_j) for j <= i (differences of log-decays), else 0,
 *   A = I + strictly-lower( beta_i (k_i . k_j) R_ij ),
 *   solve A U = diag(beta) V and A W = diag(beta exp(G)) K by forward
 *   substitution (no explicit inverse),
 *   Delta = U - W S0,
 *   O = diag(exp(G)) Q S0 + ((Q K^T) o R) Delta      (R inclusive of j = i),
 *   S_out = exp(G_n) S0 + K^T diag(exp(G_n - G_j)) Delta.
 * Same argument layout as oracle_core_sequential plus the chunk length C.
 */
int oracle_core_chunked(int T, int dk, int dv, int C, const double *q, const double *k,
                        const double *v, const double *g, const double *beta,
                        double *S, double *o)
{
    if (C < 1)
        return -1;
    size_t cc = (size_t)C;
    double *G = malloc(sizeof(double) * cc);
    double *A = malloc(sizeof(double) * cc * cc);
    double *U = malloc(sizeof(double) * cc * (size_t)dv);
    double *W = malloc(sizeof(double) * cc * (size_t)dk);
    double *Dl = malloc(sizeof(double) * cc * (size_t)dv);
    double *Sn = malloc(sizeof(double) * (size_t)dk * (size_t)dv);
    if (!G || !A || !U || !W || !Dl || !Sn) {
        free(G); free(A); free(U); free(W); free(Dl); free(Sn);
        return -1;
    }
    for (int t0 = 0; t0 < T; t0 += C) {
        int n = (T - t0 < C) ? (T - t0) : C;
        const double *Q = q + (size_t)t0 * dk, *K = k + (size_t)t0 * dk;
        const double *V = v + (size_t)t0 * dv;
        double run = 0.0;
        for (int i = 0; i < n; ++i) {
            run += g[t0 + i];
            G[i] = run;
        }
        /* strictly lower part of A */
        for (int i = 0; i < n; ++i)
            for (int j = 0; j < i; ++j) {
                double kk = 0.0;
                for (int m = 0; m < dk; ++m)
                    kk += K[(size_t)i * dk + m] * K[(size_t)j * dk + m];
                A[(size_t)i * n + j] = beta[t0 + i] * kk * exp(G[i] - G[j]);
            }
        /* forward substitution: row i of U and W */
        for (int i = 0; i < n; ++i) {
            double bi = beta[t0 + i];
            for (int c = 0; c < dv; ++c) {
                double acc = bi * V[(size_t)i * dv + c];
                for (int j = 0; j < i; ++j)
                    acc -= A[(size_t)i * n + j] * U[(size_t)j * dv + c];
                U[(size_t)i * dv + c] = acc;
            }
            double bd = bi * exp(G[i]);
            for (int c = 0; c < dk; ++c) {
                double acc = bd * K[(size_t)i * dk + c];
                for (int j = 0; j < i; ++j)
                    acc -= A[(size_t)i * n + j] * W[(size_t)j * dk + c];
                W[(size_t)i * dk + c] = acc;
            }
        }
        /* Delta = U - W S0 */
        for (int i = 0; i < n; ++i)
            for (int c = 0; c < dv; ++c) {
                double acc = U[(size_t)i * dv + c];
                for (int m = 0; m < dk; ++m)
                    acc -= W[(size_t)i * dk + m] * S[(size_t)m * dv + c];
                Dl[(size_t)i * dv + c] = acc;
            }
        /* O = diag(exp G) Q S0 + ((Q K^T) o R) Delta */
        for (int i = 0; i < n; ++i) {
            double di = exp(G[i]);
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int m = 0; m < dk; ++m)
                    acc += Q[(size_t)i * dk + m] * S[(size_t)m * dv + c];
                o[(size_t)(t0 + i) * dv + c] = di * acc;
            }
            for (int j = 0; j <= i; ++j) {
                double qk = 0.0;
                for (int m = 0; m < dk; ++m)
                    qk += Q[(size_t)i * dk + m] * K[(size_t)j * dk + m];
                double pij = qk * exp(G[i] - G[j]);
                for (int c = 0; c < dv; ++c)
                    o[(size_t)(t0 + i) * dv + c] += pij * Dl[(size_t)j * dv + c];
            }
        }
        /* S_out = exp(G_n) S0 + K^T diag(exp(G_n - G_j)) Delta */
        double dC = exp(G[n - 1]);
        for (int m = 0; m < dk; ++m)
            for (int c = 0; c < dv; ++c) {
                double acc = dC * S[(size_t)m * dv + c];
                for (int j = 0; j < n; ++j)
                    acc += K[(size_t)j * dk + m] * exp(G[n - 1] - G[j]) * Dl[(size_t)j * dv + c];
                Sn[(size_t)m * dv + c] = acc;
            }
        memcpy(S, Sn, sizeof(double) * (size_t)dk * dv);
    }
    free(G); free(A); free(U); free(W); free(Dl); free(Sn);
    return 0;
}

/* C = A B for n x n matrices (row-major). */
static void matmul_sq(int n, const double *A, const double *B, double *C)
{
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int m = 0; m < n; ++m)
                acc += A[(size_t)i * n + m] * B[(size_t)m * n + j];
            C[(size_t)i * n + j] = acc;
        }
}

/*
 * Brute-force expansion of the recurrence, used only to cross-check the other
 * two forms on tiny T.  With P_t = exp(g_t) (I - beta_t k_t k_t^T) formed as
 * explicit dk x dk matrices, the K-major state after t tokens is
 *   S_t = (P_t ... P_1) S_0 + sum_{j<=t} (P_t ... P_{j+1}) beta_j k_j v_j^T
 * (the [FE] gdn.core product S_t = e^{g_t} S_{t-1}(I - beta k k^T) + beta v k^T
 * transposed, P_t being symmetric), and o_t = S_t^T q_t.  Every S_t is rebuilt
 * from S_0 and explicit matrix products, never from S_{t-1}.
 */
int oracle_core_bruteforce(int T, int dk, int dv, const double *q, const double *k,
                           const double *v, const double *g, const double *beta,
                           double *S, double *o)
{
    size_t n2 = (size_t)dk * dk;
    double *P = malloc(sizeof(double) * n2 * (size_t)(T > 0 ? T : 1));
    double *M = malloc(sizeof(double) * n2);
    double *Tm = malloc(sizeof(double) * n2);
    double *S0 = malloc(sizeof(double) * (size_t)dk * dv);
    double *St = malloc(sizeof(double) * (size_t)dk * dv);
    if (!P || !M || !Tm || !S0 || !St) {
        free(P); free(M); free(Tm); free(S0); free(St);
        return -1;
    }
    memcpy(S0, S, sizeof(double) * (size_t)dk * dv);
    for (int t = 0; t < T; ++t) {
        double a = exp(g[t]);
        double *Pt = P + (size_t)t * n2;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dk; ++j)
                Pt[(size_t)i * dk + j] =
                    a * ((i == j ? 1.0 : 0.0) - beta[t] * k[(size_t)t * dk + i] * k[(size_t)t * dk + j]);
    }
    for (int t = 0; t < T; ++t) {
        /* M = P_t ... P_1, accumulated left-multiplying */
        for (size_t e = 0; e < n2; ++e)
            M[e] = 0.0;
        for (int i = 0; i < dk; ++i)
            M[(size_t)i * dk + i] = 1.0;
        for (int s = 0; s <= t; ++s) {
            matmul_sq(dk, P + (size_t)s * n2, M, Tm);
            memcpy(M, Tm, sizeof(double) * n2);
        }
        /* S_t = M S_0 */
        for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int m = 0; m < dk; ++m)
                    acc += M[(size_t)i * dk + m] * S0[(size_t)m * dv + c];
                St[(size_t)i * dv + c] = acc;
            }
        /* + sum_j (P_t ... P_{j+1}) beta_j k_j v_j^T */
        for (int j = 0; j <= t; ++j) {
            for (size_t e = 0; e < n2; ++e)
                M[e] = 0.0;
            for (int i = 0; i < dk; ++i)
                M[(size_t)i * dk + i] = 1.0;
            for (int s = j + 1; s <= t; ++s) {
                matmul_sq(dk, P + (size_t)s * n2, M, Tm);
                memcpy(M, Tm, sizeof(double) * n2);
            }
            for (int i = 0; i < dk; ++i) {
                double mk = 0.0;
                for (int m = 0; m < dk; ++m)
                    mk += M[(size_t)i * dk + m] * k[(size_t)j * dk + m];
                for (int c = 0; c < dv; ++c)
                    St[(size_t)i * dv + c] += beta[j] * mk * v[(size_t)j * dv + c];
            }
        }
        for (int c = 0; c < dv; ++c) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += St[(size_t)i * dv + c] * q[(size_t)t * dk + i];
            o[(size_t)t * dv + c] = acc;
        }
    }
    if (T > 0)
        memcpy(S, St, sizeof(double) * (size_t)dk * dv);
    free(P); free(M); free(Tm); free(S0); free(St);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* The whole path, in the mixer boundary's own input formats                 */
/* ------------------------------------------------------------------------ */

/* Sizes of one call, for addressing the raw inputs. */
struct layout {
    int T, Hk, Hv, dk, dv;
    size_t Cc;
};

/*
 * Raw (pre-conv) input of channel c of batch b at step tau.  Channels are
 * ordered q (Hk*dk), k (Hk*dk), v (Hv*dv).  Steps before 0 come from the conv
 * state (entry 3 + tau, oldest first) or are zero.
 */
static double raw_input(const struct layout *L, const uint16_t *q, const uint16_t *k,
                        const uint16_t *v, const uint16_t *conv_state_in, int b, size_t c,
                        int tau)
{
    size_t nq = (size_t)L->Hk * L->dk;
    if (tau < 0)
        return conv_state_in ? bf16_to_f64(conv_state_in[((size_t)b * 3 + (size_t)(3 + tau)) * L->Cc + c])
                             : 0.0;
    size_t row_qk = ((size_t)b * L->T + (size_t)tau) * L->Hk * L->dk;
    if (c < nq)
        return bf16_to_f64(q[row_qk + c]);
    if (c < 2 * nq)
        return bf16_to_f64(k[row_qk + (c - nq)]);
    size_t row_v = ((size_t)b * L->T + (size_t)tau) * L->Hv * L->dv;
    return bf16_to_f64(v[row_v + (c - 2 * nq)]);
}

/*
 * Prefill of the mixer hot path for the listed chains ([FE] gdn.conv ->
 * gdn.core -> gdn.norm; [HQ] §9.3-§9.9).
 *
 * Inputs use the boundary's layouts: q,k [B][T][Hk][dk] and v,z [B][T][Hv][dv]
 * as bf16 bits; g (log-decay), beta [B][T][Hv] fp32; conv_w [Cc][4] bf16 with
 * channels ordered q (Hk*dk), k (Hk*dk), v (Hv*dv), Cc = 2*Hk*dk + Hv*dv;
 * norm_w [dv] bf16; state_in [B][Hv][dk][dv] fp32 (NULL = zeros);
 * conv_state_in [B][3][Cc] bf16 raw pre-conv inputs of steps -3..-1 (NULL =
 * zeros).  conv_width is 0 (q,k,v used as they are, no SiLU) or 4.
 * use_norm = 0 returns the raw core read-out o instead of the gated norm.
 *
 * chains lists n_chains indices b*Hv + h (NULL = all B*Hv in order).  Outputs
 * per listed chain: y [n][T][dv] fp64, state_out [n][dk][dv] fp64.  When
 * conv_state_out is not NULL the raw inputs of the last three steps are
 * written there as bf16 bits [B][3][Cc] (entries before step 0 come from
 * conv_state_in, or are zero).  Value head h reads key head h / (Hv/Hk).
 * Returns 0, -1 on bad arguments, -2 on allocation failure.
 */
int oracle_prefill(int B, int T, int Hk, int Hv, int dk, int dv, int conv_width,
                   int use_norm, double eps_l2, double eps_norm,
                   const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   const float *g, const float *beta, const uint16_t *z,
                   const uint16_t *conv_w, const uint16_t *norm_w,
                   const float *state_in, const uint16_t *conv_state_in,
                   int n_chains, const int32_t *chains, double *y, double *state_out,
                   uint16_t *conv_state_out, int n_threads)
{
    if (B < 1 || T < 1 || Hk < 1 || Hv < 1 || dk < 1 || dv < 1 || Hv % Hk)
        return -1;
    if (conv_width != 0 && conv_width != 4)
        return -1;
    if (conv_width == 4 && !conv_w)
        return -1;
    if (use_norm && (!z || !norm_w))
        return -1;
    const int ratio = Hv / Hk;
    const size_t Cc = (size_t)2 * Hk * dk + (size_t)Hv * dv;
    const int nc = chains ? n_chains : B * Hv;
    const struct layout L = {T, Hk, Hv, dk, dv, Cc};
    int status = 0;

    if (conv_state_out && conv_width == 4) {
        for (int b = 0; b < B; ++b)
            for (int s = 0; s < 3; ++s) {
                int tau = T - 3 + s;
                for (size_t c = 0; c < Cc; ++c) {
                    uint16_t val;
                    if (tau >= 0) {
                        if (c < (size_t)Hk * dk)
                            val = q[(((size_t)b * T + tau) * Hk) * dk + c];
                        else if (c < (size_t)2 * Hk * dk)
                            val = k[(((size_t)b * T + tau) * Hk) * dk + (c - (size_t)Hk * dk)];
                        else
                            val = v[(((size_t)b * T + tau) * Hv) * dv + (c - (size_t)2 * Hk * dk)];
                    } else {
                        val = conv_state_in ? conv_state_in[((size_t)b * 3 + (size_t)(3 + tau)) * Cc + c] : 0;
                    }
                    conv_state_out[((size_t)b * 3 + s) * Cc + c] = val;
                }
            }
    }

#ifdef _OPENMP
    if (n_threads < 1)
        n_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(min : status)
#endif
    for (int ci = 0; ci < nc; ++ci) {
        int chain = chains ? chains[ci] : ci;
        if (chain < 0 || chain >= B * Hv) {
            status = -1;
            continue;
        }
        int b = chain / Hv, h = chain % Hv, kh = h / ratio;
        size_t cq0 = (size_t)kh * dk, ck0 = (size_t)Hk * dk + (size_t)kh * dk;
        size_t cv0 = (size_t)2 * Hk * dk + (size_t)h * dv;
        double *buf = malloc(sizeof(double) * ((size_t)dk * dv + 6 * (size_t)dk + 8 * (size_t)dv + 16));
        if (!buf) {
            status = -2;
            continue;
        }
        double *S = buf;
        double *uq = S + (size_t)dk * dv, *uk = uq + dk, *qh = uk + dk, *kh_ = qh + dk;
        double *tmp = kh_ + dk, *w4 = tmp + dk;               /* w4: 4 doubles   */
        double *uv = w4 + 8, *o = uv + dv, *zz = o + dv, *nw = zz + dv, *yy = nw + dv;
        double *p = yy + dv, *d = p + dv, *xs = d + dv;       /* xs: 8 doubles   */
        double sq_scale = 1.0 / sqrt((double)dk);

        if (state_in) {
            const float *src = state_in + (size_t)chain * dk * dv;
            for (size_t e = 0; e < (size_t)dk * dv; ++e)
                S[e] = (double)src[e];
        } else {
            memset(S, 0, sizeof(double) * (size_t)dk * dv);
        }
        if (use_norm)
            for (int j = 0; j < dv; ++j)
                nw[j] = bf16_to_f64(norm_w[j]);

        for (int t = 0; t < T; ++t) {
            for (int part = 0; part < 3; ++part) {
                int n = part < 2 ? dk : dv;
                size_t c0 = part == 0 ? cq0 : part == 1 ? ck0 : cv0;
                double *dst = part == 0 ? uq : part == 1 ? uk : uv;
                for (int i = 0; i < n; ++i) {
                    size_t c = c0 + (size_t)i;
                    if (conv_width == 0) {
                        dst[i] = raw_input(&L, q, k, v, conv_state_in, b, c, t);
                    } else {
                        for (int j = 0; j < 4; ++j) {
                            w4[j] = bf16_to_f64(conv_w[c * 4 + (size_t)j]);
                            xs[j] = raw_input(&L, q, k, v, conv_state_in, b, c, t + j - 3);
                        }
                        /* one-step conv: feed the window x[t-3..t] as a 4-step sequence
                           and keep its last output */
                        double u4[4];
                        oracle_conv_silu_channel(4, xs, w4, NULL, u4);
                        dst[i] = u4[3];
                    }
                }
            }
            oracle_l2norm(dk, uq, eps_l2, sq_scale, qh);
            oracle_l2norm(dk, uk, eps_l2, 1.0, kh_);
            size_t gi = ((size_t)b * T + t) * Hv + h;
            core_step(dk, dv, S, qh, kh_, uv, (double)g[gi], (double)beta[gi], o, p, d);
            double *yrow = y + ((size_t)ci * T + t) * dv;
            if (use_norm) {
                const uint16_t *zr = z + (((size_t)b * T + t) * Hv + h) * dv;
                for (int j = 0; j < dv; ++j)
                    zz[j] = bf16_to_f64(zr[j]);
                oracle_gated_rmsnorm(dv, o, zz, nw, eps_norm, yrow);
            } else {
                memcpy(yrow, o, sizeof(double) * dv);
            }
        }
        memcpy(state_out + (size_t)ci * dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(buf);
    }
    return status;
}

/*
 * One decode step ([HQ] §13.3: one recurrent step with the stored conv and
 * recurrent state): the prefill above with T = 1, reading the previous state
 * and the 3-step conv window.  q,k [B][Hk][dk]; v,z [B][Hv][dv]; g,beta
 * [B][Hv]; state [B][Hv][dk][dv] fp32; conv_state [B][3][Cc] bf16.  Outputs as
 * for oracle_prefill (y [n][dv], state_out [n][dk][dv], conv_state_out).
 */
int oracle_decode_step(int B, int Hk, int Hv, int dk, int dv, int conv_width, int use_norm,
                       double eps_l2, double eps_norm, const uint16_t *q, const uint16_t *k,
                       const uint16_t *v, const float *g, const float *beta, const uint16_t *z,
                       const uint16_t *conv_w, const uint16_t *norm_w, const float *state,
                       const uint16_t *conv_state, int n_chains, const int32_t *chains,
                       double *y, double *state_out, uint16_t *conv_state_out, int n_threads)
{
    return oracle_prefill(B, 1, Hk, Hv, dk, dv, conv_width, use_norm, eps_l2, eps_norm, q, k, v,
                          g, beta, z, conv_w, norm_w, state, conv_state, n_chains, chains, y,
                          state_out, conv_state_out, n_threads);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
