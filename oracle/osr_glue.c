/*
 * osr_glue.c -- fp64 CPU oracle for the layer glue around the Orthogonal
 * State Recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  It is the correctness reference for the GPU
 * glue kernels; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code with the HIP library.
 *
 * What it computes ("Lattice: Learning to Efficiently Compress the Memory",
 * arXiv 2504.05646, section "Experiments", paragraph on the Lattice block,
 * and the experiment-details appendix):
 *
 *   * q and k each pass through a short causal 1-D convolution of width 4
 *     along the sequence, one filter per channel (the Mamba-style block the
 *     pages adopt).  With W = 4 taps w[0..3] and bias b,
 *         out_t = b + sum_j w[j] x_{t-3+j}
 *     so w[3] weighs the current token; tokens before the sequence start are
 *     the carried history (zero at a sequence start).
 *   * the writing intensity is gamma_t = sigmoid(W_gamma x_t); the product
 *     W_gamma x_t (the logit) is the caller's, the glue applies the sigmoid.
 *   * the recurrence's output y passes through a GeLU post-gate:
 *         out = y * GeLU(g),   GeLU(x) = x Phi(x),  Phi the standard normal CDF
 *     with g the gate branch's projection (the caller's).
 *
 * Readings where the pages are silent: the convolution is depthwise, causal,
 * with a per-channel bias and no activation after it; the post-gate
 * multiplies y by GeLU of a separate projection; GeLU is the exact (erf) form.
 *
 * Arithmetic is IEEE double throughout, no fast-math.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define GLUE_W 4

/*
 * Depthwise causal convolution of one [B, T, N] sequence of channels (N =
 * H*m for q or k), with weights w [N, 4] and bias b [N] (NULL: none).
 * hist_in [B, 3, N] holds the 3 tokens before t = 0, oldest first (NULL:
 * zeros); hist_out [B, 3, N] (NULL: not written) receives the 3 tokens that
 * precede the next call, i.e. the last 3 of (hist_in, x).
 */
int oracle_glue_conv(int B, int T, int N, const double* x, const double* w, const double* b,
                     const double* hist_in, double* out, double* hist_out) {
    if (B < 0 || T < 0 || N <= 0) return -2;
    if (!x || !w || !out) return -1;
    const int P = GLUE_W - 1;
    for (int bb = 0; bb < B; ++bb) {
        for (int n = 0; n < N; ++n) {
            /* x extended by the history: xe(t) for t in [-3, T) */
            for (int t = 0; t < T; ++t) {
                double acc = b ? b[n] : 0.0;
                for (int j = 0; j < GLUE_W; ++j) {
                    const int s = t - P + j;
                    double xv;
                    if (s >= 0)
                        xv = x[((size_t)bb * T + s) * N + n];
                    else
                        xv = hist_in ? hist_in[((size_t)bb * P + (s + P)) * N + n] : 0.0;
                    acc += w[(size_t)n * GLUE_W + j] * xv;
                }
                out[((size_t)bb * T + t) * N + n] = acc;
            }
            if (hist_out) {
                for (int r = 0; r < P; ++r) {
                    const int s = T - P + r;
                    double xv;
                    if (s >= 0)
                        xv = x[((size_t)bb * T + s) * N + n];
                    else
                        xv = hist_in ? hist_in[((size_t)bb * P + (s + P)) * N + n] : 0.0;
                    hist_out[((size_t)bb * P + r) * N + n] = xv;
                }
            }
        }
    }
    return 0;
}

/* gamma = sigmoid(logit) = 1 / (1 + exp(-logit)), elementwise over n values. */
int oracle_glue_sigmoid(int64_t n, const double* logit, double* out) {
    if (n < 0) return -2;
    if (n && (!logit || !out)) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = 1.0 / (1.0 + exp(-logit[i]));
    return 0;
}

/* out = y * GeLU(g), GeLU(x) = x Phi(x), elementwise.  Phi(x) is evaluated as
 * erfc(-x / sqrt 2) / 2, which equals (1 + erf(x / sqrt 2)) / 2 but keeps its
 * relative accuracy in the negative tail, where 1 + erf cancels. */
int oracle_glue_gelu_gate(int64_t n, const double* y, const double* g, double* out) {
    if (n < 0) return -2;
    if (n && (!y || !g || !out)) return -1;
    for (int64_t i = 0; i < n; ++i) {
        const double x = g[i];
        out[i] = y[i] * (x * (0.5 * erfc(-x / sqrt(2.0))));
    }
    return 0;
}
