/*
 * mss_oracle_cplx.c -- plain fp64 CPU oracle for the selective-scan forward
 * with a complex diagonal A.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path never
 * calls it, links it or falls back to it, and it shares no code with it.
 *
 * What it computes (the plain definition, sequential in time):
 *
 *   The recurrence is the real forward's (see mss_oracle.c), carried out in
 *   complex arithmetic.  The pages note that the official CUDA kernel
 *   supports complex A with an exp2 of a complex argument written by hand
 *   (createcentury blog post reading the kernel, section "主要な最適化テクニック");
 *   they do not spell out the parameters, so this oracle takes the plainest
 *   reading consistent with the real case:
 *       A[n]   = -exp(A_log[n]) + i A_imag[n]   (decay from the real part,
 *                                                 rotation from the imaginary)
 *       a_t[n] = exp(Delta_t A[n])               (complex exponential)
 *       b_t[n] = Delta_t B_t[n] u_t              (B complex, u real)
 *       h_t[n] = a_t[n] h_{t-1}[n] + b_t[n]      (complex state)
 *       y_t    = Re(sum_n C_t[n] h_t[n]) + D u_t, then y_t *= silu(z_t)
 *   Delta, D, z and the gate are as in the real forward.
 *
 * Layouts (contiguous, row-major; complex values as (re, im) double pairs):
 *   u, delta_raw, z, out : [batch][dim][seqlen]           real
 *   B, C                 : [batch][dstate][seqlen]        complex
 *   A_log, A_imag        : [dim][dstate]                  real
 *   D, dt_bias           : [dim]                          real
 *   h0, final_state      : [batch][dim][dstate]           complex
 * Nullable: D, z, dt_bias, h0 (-> 0 / no gate), final_state (-> not written).
 */
#include <complex.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

double mss_oracle_softplus(double x);
double mss_oracle_silu(double x);

int mss_oracle_scan_fwd_complex(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate,
                                const double *u, const double *delta_raw, const double *A_log,
                                const double *A_imag, const double *B_ri, const double *C_ri,
                                const double *D, const double *z, const double *dt_bias,
                                const double *h0_ri, int delta_softplus, double *out,
                                double *final_ri, int nthreads) {
    if (dstate < 1 || dstate > 256) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const double complex *B = (const double complex *)B_ri;
    const double complex *C = (const double complex *)C_ri;
    const double complex *h0 = (const double complex *)h0_ri;
    double complex *final_state = (double complex *)final_ri;
    int64_t nchan = batch * dim;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ch = 0; ch < nchan; ++ch) {
        int64_t b = ch / dim;
        int64_t d = ch % dim;
        double complex A[256];
        double complex h[256];
        for (int64_t n = 0; n < dstate; ++n) {
            A[n] = -exp(A_log[d * dstate + n]) + I * A_imag[d * dstate + n];
            h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;
        }
        double bias = dt_bias ? dt_bias[d] : 0.0;
        double skip = D ? D[d] : 0.0;
        for (int64_t t = 0; t < seqlen; ++t) {
            double x = delta_raw[(b * dim + d) * seqlen + t] + bias;
            double delta = delta_softplus ? mss_oracle_softplus(x) : x;
            double ut = u[(b * dim + d) * seqlen + t];
            double complex y = 0.0;
            for (int64_t n = 0; n < dstate; ++n) {
                double complex a = cexp(delta * A[n]);
                double complex bt = delta * B[(b * dstate + n) * seqlen + t] * ut;
                h[n] = a * h[n] + bt;
                y += C[(b * dstate + n) * seqlen + t] * h[n];
            }
            double yr = creal(y) + skip * ut;
            if (z) yr *= mss_oracle_silu(z[(b * dim + d) * seqlen + t]);
            out[(b * dim + d) * seqlen + t] = yr;
        }
        if (final_state)
            for (int64_t n = 0; n < dstate; ++n) final_state[(b * dim + d) * dstate + n] = h[n];
    }
    return 0;
}
