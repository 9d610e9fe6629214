/*
 * mss_oracle_bwd.c -- plain fp64 CPU oracle for the backward pass of the
 * selective-scan forward in mss_oracle.c.
 *
 * TEST INFRASTRUCTURE ONLY, like mss_oracle.c: only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load it.  It shares no code,
 * header, helper or constant with the HIP path.
 *
 * The pages name the training backward as the missing piece ("mamba-metal:
 * Apple Silicon で Mamba を動かす", section "残り課題").  What it must compute
 * follows from the forward alone (the recurrence of section "Selective scan
 * の本質", the per-state discretisation of the decode equation in section
 * "O(L) インクリメンタルデコード", the skip and z gate of createcentury's
 * reading of the CUDA kernel, section "1チャンク内の処理フロー", and the fused
 * softplus and -exp(A_log) of the SpeechLens notes): given the gradient dout
 * of a scalar loss with respect to out (and, optionally, dfinal with respect
 * to the exported final state), return the gradient with respect to every
 * input.  The chain rule applied to the forward, step by step in reverse time:
 *
 *   forward (per channel b,d):  x_t = delta_raw_t + dt_bias,  Delta_t = softplus(x_t) or x_t,
 *       A_n = -exp(A_log[d,n]),  a_tn = exp(Delta_t A_n),
 *       h_tn = a_tn h_(t-1)n + Delta_t B_tn u_t   (h_(-1) = h0),
 *       y_t = sum_n C_tn h_tn + D u_t,  out_t = y_t silu(z_t) (or y_t)
 *   reverse: g_n carries dLoss/dh_(t)n from the future (g = dfinal at t = L-1)
 *       dy_t   = dout_t silu(z_t)                  dz_t = dout_t y_t silu'(z_t)
 *       G_tn   = g_n + dy_t C_tn                   (total adjoint of h_tn)
 *       dC_tn += dy_t h_tn                         dB_tn += G_tn Delta_t u_t
 *       du_t   = dy_t D + sum_n G_tn B_tn Delta_t
 *       dDelta = sum_n G_tn B_tn u_t + sum_n G_tn h_(t-1)n a_tn A_n
 *       dA_n  += G_tn h_(t-1)n a_tn Delta_t        g_n = G_tn a_tn
 *       ddelta_raw_t = dDelta sigmoid(x_t) (softplus' = sigmoid) or dDelta
 *   and after the walk: dh0 = g, dA_log = dA A (since dA/dA_log = A),
 *   dD = sum_t dy_t u_t, ddt_bias = sum_t ddelta_raw_t, dB and dC summed over
 *   the channels that share them, dA_log, dD and ddt_bias over the batch.
 *
 * Layouts as in mss_oracle.c (fp64, contiguous): u, delta_raw, z, dout and
 * the per-element gradients [batch][dim][seqlen]; B, C, dB, dC
 * [batch][dstate][seqlen]; A_log, dA_log [dim][dstate]; D, dt_bias, dD,
 * ddt_bias [dim]; h0, dfinal, dh0 [batch][dim][dstate].
 * Nullable inputs: D, z, dt_bias, h0, dfinal (each as 0 / absent).
 * Nullable outputs: dD, dz, ddt_bias, dh0 (not written).
 * Every gradient is overwritten (the sums start from zero).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

double mss_oracle_softplus(double x); /* mss_oracle.c */
double mss_oracle_silu(double z);     /* mss_oracle.c */

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* d silu / dz = sigmoid(z) (1 + z (1 - sigmoid(z))) */
static double silu_grad(double z) {
    double s = sigmoid(z);
    return s * (1.0 + z * (1.0 - s));
}

int mss_oracle_scan_bwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate,
                        const double *u, const double *delta_raw, const double *A_log,
                        const double *B, const double *C, const double *D, const double *z,
                        const double *dt_bias, const double *h0, int delta_softplus,
                        const double *dout, const double *dfinal,
                        double *du, double *ddelta_raw, double *dA_log, double *dB, double *dC,
                        double *dD, double *dz, double *ddt_bias, double *dh0) {
    if (dstate < 1 || dstate > 256 || seqlen < 1) return -1;
    memset(dA_log, 0, sizeof(double) * dim * dstate);
    memset(dB, 0, sizeof(double) * batch * dstate * seqlen);
    memset(dC, 0, sizeof(double) * batch * dstate * seqlen);
    if (dD) memset(dD, 0, sizeof(double) * dim);
    if (ddt_bias) memset(ddt_bias, 0, sizeof(double) * dim);
    /* hist[t + 1][n] = h_t[n], hist[0][n] = h_(-1)[n] */
    double *hist = malloc(sizeof(double) * (seqlen + 1) * dstate);
    double *delta = malloc(sizeof(double) * seqlen);
    if (!hist || !delta) {
        free(hist);
        free(delta);
        return -2;
    }
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const int64_t row = (b * dim + d) * seqlen;
            const double *B_b = B + b * dstate * seqlen;
            const double *C_b = C + b * dstate * seqlen;
            double A[256], g[256], dA[256];
            double bias = dt_bias ? dt_bias[d] : 0.0;
            double skip = D ? D[d] : 0.0;
            for (int64_t n = 0; n < dstate; ++n) {
                A[n] = -exp(A_log[d * dstate + n]);
                hist[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;
                dA[n] = 0.0;
            }
            /* forward, keeping every state */
            for (int64_t t = 0; t < seqlen; ++t) {
                double x = delta_raw[row + t] + bias;
                delta[t] = delta_softplus ? mss_oracle_softplus(x) : x;
                for (int64_t n = 0; n < dstate; ++n)
                    hist[(t + 1) * dstate + n] = exp(delta[t] * A[n]) * hist[t * dstate + n] +
                                                 delta[t] * B_b[n * seqlen + t] * u[row + t];
            }
            /* reverse */
            for (int64_t n = 0; n < dstate; ++n)
                g[n] = dfinal ? dfinal[(b * dim + d) * dstate + n] : 0.0;
            double sum_dy_u = 0.0, sum_dx = 0.0;
            for (int64_t t = seqlen - 1; t >= 0; --t) {
                double x = delta_raw[row + t] + bias;
                double ut = u[row + t];
                const double *h_t = hist + (t + 1) * dstate;
                const double *h_prev = hist + t * dstate;
                double dy = dout[row + t];
                if (z) {
                    double y = skip * ut;
                    for (int64_t n = 0; n < dstate; ++n) y += C_b[n * seqlen + t] * h_t[n];
                    if (dz) dz[row + t] = dout[row + t] * y * silu_grad(z[row + t]);
                    dy = dout[row + t] * mss_oracle_silu(z[row + t]);
                }
                sum_dy_u += dy * ut;
                double du_t = dy * skip;
                double ddelta = 0.0;
                for (int64_t n = 0; n < dstate; ++n) {
                    double Bn = B_b[n * seqlen + t];
                    double G = g[n] + dy * C_b[n * seqlen + t];
                    dC[b * dstate * seqlen + n * seqlen + t] += dy * h_t[n];
                    dB[b * dstate * seqlen + n * seqlen + t] += G * delta[t] * ut;
                    du_t += G * Bn * delta[t];
                    ddelta += G * Bn * ut;
                    double a = exp(delta[t] * A[n]);
                    double ga = G * h_prev[n] * a;
                    ddelta += ga * A[n];
                    dA[n] += ga * delta[t];
                    g[n] = G * a;
                }
                du[row + t] = du_t;
                double dx = delta_softplus ? ddelta * sigmoid(x) : ddelta;
                ddelta_raw[row + t] = dx;
                sum_dx += dx;
            }
            for (int64_t n = 0; n < dstate; ++n) {
                dA_log[d * dstate + n] += dA[n] * A[n];
                if (dh0) dh0[(b * dim + d) * dstate + n] = g[n];
            }
            if (dD) dD[d] += sum_dy_u;
            if (ddt_bias) ddt_bias[d] += sum_dx;
        }
    }
    free(hist);
    free(delta);
    return 0;
}
