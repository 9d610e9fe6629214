/*
 * mss_oracle.c -- plain fp64 CPU oracle for the Mamba selective-scan forward
 * and its one-token state update.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (libmss and its Python binding) never calls it, links it or falls back to it.
 * It shares no code, header, helper or constant with the HIP path.
 *
 * What it computes (the plain definition, evaluated sequentially in time):
 *
 *   Mamba's hidden state follows the input-dependent linear recurrence
 *       h_t = Abar_t * h_{t-1} + Bbar_t * u_t,     y_t = C_t . h_t
 *   with Abar_t = exp(Delta_t * A) for a diagonal A
 *   ("mamba-metal: Apple Silicon で Mamba を動かす", section
 *   "Selective scan の本質", the recurrence equation).
 *
 *   Per diagonal entry n the discretisation used is
 *       a_t[n] = exp(Delta_t * A[n]),   b_t[n] = Delta_t * B_t[n] * u_t
 *   (createcentury blog post reading the official CUDA kernel, section
 *   "なぜ「scan」か", the thread_data pair; and the decode-step equation in
 *   "mamba-metal", section "O(L) インクリメンタルデコード").
 *
 *   Delta_t = softplus(delta_raw_t + dt_bias) when softplus is on, else
 *   delta_raw_t + dt_bias; A = -exp(A_log)
 *   (SpeechLens kernel-optimization notes, selective-scan section: softplus
 *   and -exp(A_log) fused into the scan).
 *
 *   y_t = sum_n C_t[n] h_t[n] + D * u_t, then y_t *= z_t * sigmoid(z_t)
 *   (CUDA-kernel post, section "1チャンク内の処理フロー", steps 3, 4e and 6).
 *
 *   Every channel (b, d) is independent; time is sequential inside a channel.
 *   The state starts at h0 (or 0) and the state after the last step is
 *   returned (the final-state hand-off named in "mamba-metal", section
 *   "残り課題").
 *
 * Layouts (all contiguous, row-major, fp64):
 *   u, delta_raw, z, out : [batch][dim][seqlen]
 *   B, C                 : [batch][dstate][seqlen]
 *   A_log                : [dim][dstate]
 *   D, dt_bias           : [dim]
 *   h0, final_state      : [batch][dim][dstate]
 * Nullable: D (-> 0), z (-> no gate), dt_bias (-> 0), h0 (-> 0),
 *           final_state (-> not written).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(x) = log(1 + e^x), written in the form that neither overflows for
 * large x nor cancels for very negative x: max(x, 0) + log1p(e^-|x|).  The two
 * forms are equal as real numbers. */
double mss_oracle_softplus(double x) {
    double m = x > 0.0 ? x : 0.0;
    return m + log1p(exp(-fabs(x)));
}

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z). */
double mss_oracle_silu(double z) {
    return z / (1.0 + exp(-z));
}

static double discretised_delta(double delta_raw, double bias, int delta_softplus) {
    double x = delta_raw + bias;
    return delta_softplus ? mss_oracle_softplus(x) : x;
}

int mss_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Selective-scan forward over full sequences.  nthreads <= 0 uses the OpenMP
 * default.  Returns 0, or -1 when dstate exceeds the local state buffer. */
int mss_oracle_scan_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate,
                        const double *u, const double *delta_raw, const double *A_log,
                        const double *B, const double *C, const double *D,
                        const double *z, const double *dt_bias, const double *h0,
                        int delta_softplus, double *out, double *final_state,
                        int nthreads) {
    if (dstate < 1 || dstate > 256) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int64_t nchan = batch * dim;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ch = 0; ch < nchan; ++ch) {
        int64_t b = ch / dim;
        int64_t d = ch % dim;
        double A[256];
        double h[256];
        for (int64_t n = 0; n < dstate; ++n) {
            A[n] = -exp(A_log[d * dstate + n]);
            h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;
        }
        double bias = dt_bias ? dt_bias[d] : 0.0;
        double skip = D ? D[d] : 0.0;
        const double *u_row = u + (b * dim + d) * seqlen;
        const double *dr_row = delta_raw + (b * dim + d) * seqlen;
        const double *z_row = z ? z + (b * dim + d) * seqlen : NULL;
        const double *B_b = B + b * dstate * seqlen;
        const double *C_b = C + b * dstate * seqlen;
        double *out_row = out + (b * dim + d) * seqlen;
        for (int64_t t = 0; t < seqlen; ++t) {
            double delta = discretised_delta(dr_row[t], bias, delta_softplus);
            double ut = u_row[t];
            double y = 0.0;
            for (int64_t n = 0; n < dstate; ++n) {
                double a = exp(delta * A[n]);
                double bt = delta * B_b[n * seqlen + t] * ut;
                h[n] = a * h[n] + bt;
                y += C_b[n * seqlen + t] * h[n];
            }
            y += skip * ut;
            if (z_row) y *= mss_oracle_silu(z_row[t]);
            out_row[t] = y;
        }
        if (final_state)
            for (int64_t n = 0; n < dstate; ++n)
                final_state[(b * dim + d) * dstate + n] = h[n];
    }
    return 0;
}

/* One-token state update (decode step), written on its own: for every
 * channel, advance the state by one step in place and return that step's
 * output ("mamba-metal", section "O(L) インクリメンタルデコード", the
 * per-step equation, closed by the z gate).
 *   state               : [batch][dim][dstate], updated in place
 *   u, delta_raw, z, out: [batch][dim]
 *   B, C                : [batch][dstate]                                    */
int mss_oracle_state_update(int64_t batch, int64_t dim, int64_t dstate, double *state,
                            const double *u, const double *delta_raw, const double *A_log,
                            const double *B, const double *C, const double *D,
                            const double *z, const double *dt_bias, int delta_softplus,
                            double *out) {
    if (dstate < 1) return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            double delta = discretised_delta(delta_raw[b * dim + d],
                                             dt_bias ? dt_bias[d] : 0.0, delta_softplus);
            double x = u[b * dim + d];
            double *h = state + (b * dim + d) * dstate;
            double y = 0.0;
            for (int64_t n = 0; n < dstate; ++n) {
                double decay = exp(delta * -exp(A_log[d * dstate + n]));
                h[n] = decay * h[n] + delta * x * B[b * dstate + n];
                y += h[n] * C[b * dstate + n];
            }
            y += (D ? D[d] : 0.0) * x;
            if (z) y *= mss_oracle_silu(z[b * dim + d]);
            out[b * dim + d] = y;
        }
    }
    return 0;
}
