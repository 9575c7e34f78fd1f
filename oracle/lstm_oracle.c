/*
 * lstm_oracle.c -- plain fp64 CPU reference of the multi-layer, optionally
 * bidirectional LSTM forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header, table or helper with the HIP library
 * under layer_lstm_forward_amd/csrc, and neither side includes the other.
 *
 * What it computes (every step follows a passage of the source pages):
 *
 *   - The cell: warp-nn "Long Short-Term Memory (LSTM)", the equation block
 *     under the class signature.  Per layer and time step
 *         i = sigma(W_ii x + b_ii + W_hi h + b_hi)
 *         f = sigma(W_if x + b_if + W_hf h + b_hf)
 *         g = tanh (W_ig x + b_ig + W_hg h + b_hg)
 *         o = sigma(W_io x + b_io + W_ho h + b_ho)
 *         c' = f*c + i*g ,   h' = o*tanh(c')
 *     with sigma(z) = 1/(1+exp(-z)).
 *   - Stacked weights: the same page's "Learnable parameters" table stores
 *     the four gates as row blocks [i; f; g; o] of one (4H x in) matrix and
 *     one (4H x H) matrix, plus two bias vectors of length 4H.  The MXNet
 *     blog "LSTM Forward Computation", section "Basic Operators", describes
 *     the same concatenation, and its "MXNet Implementation" slices the
 *     result in the order in, forget, transform, out.
 *   - Two biases, both added: the warp-nn table (bias_ih, bias_hh) and the
 *     two FullyConnected ops with their own bias in "MXNet Implementation".
 *   - Time loop: "Loop Unroll" in the MXNet blog; the initial state is zero
 *     unless given ("Complete Trace: nn.LSTM", Step 1, forward()).
 *   - Layer stacking: the warp-nn symbol list says layer k > 0 takes the
 *     previous layer's output at time t; "Stack Multiple RNN Cells" in the
 *     MXNet blog keeps each layer's final state and feeds only the output
 *     sequence upward.
 *   - Bidirectional: warp-nn, the paragraph after the equations -- the
 *     reverse direction scans from the last element to the first with its
 *     own parameters, and the two directions' hidden states are concatenated
 *     with the forward one first.  Reading taken where the page is silent:
 *     the reverse output is stored at the time index of the input it has
 *     just consumed, and its "final" state is the one after consuming t = 0.
 *   - Shapes of the returned tensors: warp-nn __call__ "Returns".
 *   - Variable-length batches (oracle_lstm_forward_lengths): "Complete
 *     Trace: nn.LSTM", Step 3, lists a packed-sequence overload beside the
 *     padded one, and the MXNet blog's "Sequence Buckets" pads sequences of
 *     different lengths and ignores the padded elements.  Reading taken: with
 *     a length per batch row on the padded [T][B] layout, row b takes part
 *     only in the steps with t < len_b; elsewhere its state is left as it is
 *     and its output is zero.  Its final state is therefore the one after
 *     its last valid step, and the reverse direction starts at t = len_b - 1
 *     from the initial state.
 *
 * Layouts (all row-major, contiguous, fp64):
 *   x    [T][B][I]                   input sequence, time-major
 *   h0   [L*D][B][H] or NULL (zeros) index l*D + d, forward before reverse
 *   c0   [L*D][B][H] or NULL (zeros)
 *   params: for l in 0..L-1, for d in 0..D-1:
 *       W_ih [4H][in_l]  (in_0 = I, in_l = D*H for l > 0)
 *       W_hh [4H][H]
 *       b_ih [4H], b_hh [4H]          only when has_bias != 0
 *   y    [T][B][D*H]                 last layer's hidden states
 *   h_n  [L*D][B][H], c_n [L*D][B][H]
 *
 * nthreads > 1 splits the independent output elements of one step (batch
 * rows x gate rows, and batch rows x units) across OpenMP threads.  Each
 * element is still summed in the same order, so the result does not depend
 * on the thread count.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* time index t is past row b's sequence (variable-length batches only) */
#define PADDED(t, b) (lengths && (t) >= lengths[b])

/* Returns 0 on success, -1 on a bad argument, -2 if memory runs out.
 * lengths: NULL (every row has T steps) or B values in 1..T. */
int oracle_lstm_forward_lengths(int T, int B, int I, int H, int L, int D,
                                const double *x, const int *lengths,
                                const double *h0, const double *c0,
                                const double *const *params, int has_bias,
                                double *y, double *h_n, double *c_n, int nthreads)
{
    if (T < 1 || B < 1 || I < 1 || H < 1 || L < 1 || (D != 1 && D != 2) ||
        !x || !params || !y)
        return -1;
    if (lengths)
        for (int b = 0; b < B; ++b)
            if (lengths[b] < 1 || lengths[b] > T) return -1;
    if (nthreads < 1) nthreads = 1;
    const int per = has_bias ? 4 : 2;
    const int G = 4 * H;
    const size_t seq_out = (size_t)T * B * D * H;

    double *Y = NULL;
    double *h = malloc(sizeof(double) * (size_t)B * H);
    double *c = malloc(sizeof(double) * (size_t)B * H);
    double *pre = malloc(sizeof(double) * (size_t)B * G);
    double *Yl = malloc(sizeof(double) * seq_out);
    double *Xl = (L > 1) ? malloc(sizeof(double) * seq_out) : NULL;
    if (!h || !c || !pre || !Yl || (L > 1 && !Xl)) {
        free(h); free(c); free(pre); free(Yl); free(Xl);
        return -2;
    }

    const double *in_seq = x;
    int in_w = I;
    for (int l = 0; l < L; ++l) {
        Y = Yl;
        memset(Y, 0, sizeof(double) * seq_out);
        for (int d = 0; d < D; ++d) {
            const double *const *p = params + (size_t)(l * D + d) * per;
            const double *W_ih = p[0], *W_hh = p[1];
            const double *b_ih = has_bias ? p[2] : NULL;
            const double *b_hh = has_bias ? p[3] : NULL;
            const size_t st = (size_t)(l * D + d) * B * H;
            for (size_t e = 0; e < (size_t)B * H; ++e) {
                h[e] = h0 ? h0[st + e] : 0.0;
                c[e] = c0 ? c0[st + e] : 0.0;
            }
            for (int s = 0; s < T; ++s) {
                const int t = (d == 0) ? s : T - 1 - s;
                /* pre-activations of all four gates from the previous h */
#pragma omp parallel for collapse(2) num_threads(nthreads) if (nthreads > 1)
                for (int b = 0; b < B; ++b) {
                    for (int r = 0; r < G; ++r) {
                        if (PADDED(t, b)) continue;
                        const double *xt = in_seq + ((size_t)t * B + b) * in_w;
                        const double *wi = W_ih + (size_t)r * in_w;
                        const double *wh = W_hh + (size_t)r * H;
                        const double *hb = h + (size_t)b * H;
                        double acc = 0.0;
                        if (has_bias) acc = b_ih[r] + b_hh[r];
                        for (int k = 0; k < in_w; ++k) acc += wi[k] * xt[k];
                        for (int k = 0; k < H; ++k) acc += wh[k] * hb[k];
                        pre[(size_t)b * G + r] = acc;
                    }
                }
                /* gates, cell update and output; h of the previous step has
                 * been consumed in full above before it is overwritten here */
#pragma omp parallel for collapse(2) num_threads(nthreads) if (nthreads > 1)
                for (int b = 0; b < B; ++b) {
                    for (int j = 0; j < H; ++j) {
                        /* a padded step leaves the state alone; y stays 0 */
                        if (PADDED(t, b)) continue;
                        const double *pb = pre + (size_t)b * G;
                        const double ig = sigmoid(pb[j]);
                        const double fg = sigmoid(pb[H + j]);
                        const double gg = tanh(pb[2 * H + j]);
                        const double og = sigmoid(pb[3 * H + j]);
                        const size_t e = (size_t)b * H + j;
                        const double cn = fg * c[e] + ig * gg;
                        const double hn = og * tanh(cn);
                        c[e] = cn;
                        h[e] = hn;
                        Y[((size_t)t * B + b) * (size_t)(D * H) + (size_t)d * H + j] = hn;
                    }
                }
            }
            if (h_n) memcpy(h_n + st, h, sizeof(double) * (size_t)B * H);
            if (c_n) memcpy(c_n + st, c, sizeof(double) * (size_t)B * H);
        }
        /* the next layer reads this layer's whole output sequence */
        if (l + 1 < L) {
            double *tmp = Xl; Xl = Yl; Yl = tmp;
            in_seq = Xl;
            in_w = D * H;
        }
    }
    memcpy(y, Y, sizeof(double) * seq_out);
    free(h); free(c); free(pre); free(Yl); free(Xl);
    return 0;
}

/* Every row has all T steps. */
int oracle_lstm_forward(int T, int B, int I, int H, int L, int D,
                        const double *x, const double *h0, const double *c0,
                        const double *const *params, int has_bias,
                        double *y, double *h_n, double *c_n, int nthreads)
{
    return oracle_lstm_forward_lengths(T, B, I, H, L, D, x, NULL, h0, c0, params, has_bias,
                                       y, h_n, c_n, nthreads);
}

/* Number of threads OpenMP would use by default (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
