/*
 * mss_oracle_conv.c -- plain fp64 CPU oracle for the causal depthwise conv1d
 * (with its optional SiLU) that feeds the selective scan, and for its
 * one-token sliding-window update.
 *
 * TEST INFRASTRUCTURE ONLY, like mss_oracle.c: only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load it.  It shares no code,
 * header, helper or constant with the HIP path.
 *
 * What it computes (the plain definition, one output at a time):
 *
 *   Each channel d is filtered on its own (depthwise: as many groups as
 *   channels) with a kernel of `width` taps, causally: the output at step t
 *   sees the input at steps t-width+1 .. t only, and the input is extended to
 *   the left by width-1 samples that are zero unless a carried window is
 *   given (SpeechLens kernel-optimization notes, causal depthwise convolution
 *   section and its contract table: kernel size 4, depthwise grouping, three
 *   zero samples on the causal left edge, output length = input length).
 *   Tap k multiplies the sample k steps after the oldest one, as in a
 *   framework Conv1d (a cross-correlation):
 *       pre[b,d,t] = bias[d] + sum_{k=0}^{width-1} w[d,k] * x~[b,d,t-(width-1)+k]
 *       out[b,d,t] = silu(pre) when the activation is on, else pre
 *   (the block order in_proj -> conv1d -> SiLU of "mamba-metal: Apple
 *   Silicon で Mamba を動かす", section "カーネルから推論まで"; SpeechLens:
 *   the Conv-SiLU fusion measured in its fusion table).
 *   x~[tau] = x[tau] for tau >= 0; for tau < 0 it is init[b,d,width-1+tau]
 *   when a carried window `init` is given, else 0.
 *
 *   The decode step carries the sliding window of the last width-1 inputs
 *   between calls ("mamba-metal", section "O(L) インクリメンタルデコード":
 *   the conv1d sliding window is carried across calls).  One step appends
 *   x_t to the window, produces the output of the full width-sample window,
 *   and drops the oldest sample.
 *
 * Layouts (all contiguous, row-major, fp64):
 *   x, out              : [batch][dim][seqlen]
 *   w                   : [dim][width]
 *   bias                : [dim]               (nullable -> 0)
 *   init, final, state  : [batch][dim][width-1], oldest sample first
 *                                             (init nullable -> zeros;
 *                                              final nullable -> not written)
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

double mss_oracle_silu(double z); /* defined in mss_oracle.c */

/* x~ of the definition above: a sample of the carried window for tau < 0. */
static double extended_sample(const double *x_row, const double *init_row, int64_t width,
                              int64_t tau) {
    if (tau >= 0) return x_row[tau];
    return init_row ? init_row[width - 1 + tau] : 0.0;
}

/* Causal depthwise conv1d over full sequences.  Returns 0, or -1 for a width
 * below 1. */
int mss_oracle_conv1d_fwd(int64_t batch, int64_t dim, int64_t seqlen, int64_t width,
                          const double *x, const double *w, const double *bias,
                          const double *init, int silu, double *out, double *final) {
    if (width < 1) return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const double *x_row = x + (b * dim + d) * seqlen;
            const double *init_row = init ? init + (b * dim + d) * (width - 1) : NULL;
            const double *w_row = w + d * width;
            double *out_row = out + (b * dim + d) * seqlen;
            for (int64_t t = 0; t < seqlen; ++t) {
                double pre = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < width; ++k)
                    pre += w_row[k] * extended_sample(x_row, init_row, width, t - (width - 1) + k);
                out_row[t] = silu ? mss_oracle_silu(pre) : pre;
            }
            /* the window after the last step: the last width-1 samples of x~ */
            if (final)
                for (int64_t j = 0; j < width - 1; ++j)
                    final[(b * dim + d) * (width - 1) + j] =
                        extended_sample(x_row, init_row, width, seqlen - (width - 1) + j);
        }
    }
    return 0;
}

/* One decode step of the conv1d, written on its own: window = the carried
 * width-1 samples followed by x_t; out = act(bias + w . window); the state
 * becomes the window without its oldest sample.
 *   state : [batch][dim][width-1], updated in place
 *   x, out: [batch][dim]                                                    */
int mss_oracle_conv1d_update(int64_t batch, int64_t dim, int64_t width, double *state,
                             const double *x, const double *w, const double *bias, int silu,
                             double *out) {
    if (width < 1) return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            double *s = state + (b * dim + d) * (width - 1);
            double window[64];
            if (width > 64) return -1;
            for (int64_t k = 0; k + 1 < width; ++k) window[k] = s[k];
            window[width - 1] = x[b * dim + d];
            double pre = bias ? bias[d] : 0.0;
            for (int64_t k = 0; k < width; ++k) pre += w[d * width + k] * window[k];
            out[b * dim + d] = silu ? mss_oracle_silu(pre) : pre;
            for (int64_t k = 0; k + 1 < width; ++k) s[k] = window[k + 1];
        }
    }
    return 0;
}
