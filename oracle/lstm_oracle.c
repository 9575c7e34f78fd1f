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
 *   - Backward pass (oracle_lstm_backward): the trace page's "cuDNN
 *     Backward" section returns the gradients of the input, of the initial
 *     states and of the weights from the gradients of (output, h_n, c_n) and
 *     the activations saved by the forward; the pulsatrix "LSTMModule"
 *     reference describes backpropagation through time across the four gates
 *     and the cell carry, accumulating every weight and bias gradient over
 *     all time steps.  The gradients are those of the cell equations above by
 *     the chain rule, taken step by step in the reverse of each direction's
 *     scan order (written out in the function).
 *   - Variable-length batches (oracle_lstm_forward_lengths): "Complete
 *     Trace: nn.LSTM", Step 3, lists a packed-sequence overload beside the
 *     padded one, and the MXNet blog's "Sequence Buckets" pads sequences of
 *     different lengths and ignores the padded elements.  Reading taken: with
 *     a length per batch row on the padded [T][B] layout, row b takes part
 *     only in the steps with t < len_b; elsewhere its state is left as it is
 *     and its output is zero.  Its final state is therefore the one after
 *     its last valid step, and the reverse direction starts at t = len_b - 1
 *     from the initial state.
 *   - Dropout between layers in training (oracle_lstm_forward_dropout and
 *     the p argument of oracle_lstm_backward): the trace page's Performance
 *     Notes apply dropout to the input of every layer above the first during
 *     training only, and the op signature of its Step 3 carries the
 *     probability.  Reading taken: element e of layer l's output sequence
 *     ([T][B][D*H], time-major flat index) reaches layer l + 1 as
 *     y[e] / (1 - p) when kept and 0 when dropped (all dropped when p = 1).
 *     The draw is a counter-based generator, Philox4x64-10 (Salmon, Moraes,
 *     Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011),
 *     written here from its published definition: the block with counter
 *     (e / 4, l, call, 0) and key (seed, 0) gives four 64-bit words; word
 *     e % 4, as u = (word >> 11) * 2^-53, keeps e when u >= p.
 *
 *   - Other recurrent modes (oracle_rnn_forward): the trace page's RNNBase
 *     ("Complete Trace: nn.LSTM", Step 1) takes a mode among 'LSTM', 'GRU',
 *     'RNN_TANH' and 'RNN_RELU' but gives only the LSTM's equations.  Reading
 *     taken: the definitions of the framework whose RNNBase that page
 *     reproduces.  With gi = W_ih x_t + b_ih and gh = W_hh h + b_hh split
 *     into H-row blocks (GRU: [r; z; n], RNN: one block):
 *         GRU:  r = sigma(gi_r + gh_r),  z = sigma(gi_z + gh_z),
 *               n = tanh(gi_n + r * gh_n),  h' = (1 - z) * n + z * h
 *         RNN_TANH: h' = tanh(gi + gh);  RNN_RELU: h' = max(0, gi + gh)
 *     Stacking, directions and shapes as for the LSTM, with 3H (GRU) or H
 *     (RNN) gate rows instead of 4H and no cell state.
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
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* Philox4x64-10: ten rounds of two 64x64 -> 128-bit products on counter
 * words 0 and 2, each round mixing the high halves with the other counter
 * words and the key, the key advanced by the two Weyl constants between
 * rounds (the constants are the published ones). */
static void philox_mul(uint64_t a, uint64_t b, uint64_t *hi, uint64_t *lo)
{
    const unsigned __int128 p = (unsigned __int128)a * b;
    *hi = (uint64_t)(p >> 64);
    *lo = (uint64_t)p;
}

void oracle_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4])
{
    uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t hi0, lo0, hi1, lo1;
        philox_mul(0xD2E7470EE14C6C93ull, c0, &hi0, &lo0);
        philox_mul(0xCA5A826395121157ull, c2, &hi1, &lo1);
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += 0x9E3779B97F4A7C15ull;
        k1 += 0xBB67AE8584CAA73Bull;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Is element e of layer l's output kept by the dropout draw of call `call`? */
static int dropout_keeps(double p, uint64_t seed, uint64_t call, int l, size_t e)
{
    const uint64_t ctr[4] = {(uint64_t)(e / 4), (uint64_t)l, call, 0};
    const uint64_t key[2] = {seed, 0};
    uint64_t w[4];
    oracle_philox4x64_10(ctr, key, w);
    const double u = (double)(w[e % 4] >> 11) * 0x1p-53;
    return u >= p;
}

/* keep decisions of elements 0..n-1 of layer l's output (1 kept, 0 dropped) */
void oracle_dropout_keep(double p, uint64_t seed, uint64_t call, int l, size_t n, unsigned char *keep)
{
    for (size_t e = 0; e < n; ++e) keep[e] = (unsigned char)dropout_keeps(p, seed, call, l, e);
}

/* factor that element e of layer l's output carries into layer l + 1 */
static double dropout_factor(double p, uint64_t seed, uint64_t call, int l, size_t e)
{
    if (p <= 0.0) return 1.0;
    return dropout_keeps(p, seed, call, l, e) ? 1.0 / (1.0 - p) : 0.0;
}

/* time index t is past row b's sequence (variable-length batches only) */
#define PADDED(t, b) (lengths && (t) >= lengths[b])

/* Returns 0 on success, -1 on a bad argument, -2 if memory runs out.
 * lengths: NULL (every row has T steps) or B values in 1..T.
 * drop_p in [0, 1]: dropout between layers (0: none), drawn for (seed, call). */
static int forward_core(int T, int B, int I, int H, int L, int D,
                        const double *x, const int *lengths,
                        const double *h0, const double *c0,
                        const double *const *params, int has_bias,
                        double drop_p, uint64_t seed, uint64_t call,
                        double *y, double *h_n, double *c_n, int nthreads)
{
    if (T < 1 || B < 1 || I < 1 || H < 1 || L < 1 || (D != 1 && D != 2) ||
        !x || !params || !y || !(drop_p >= 0.0 && drop_p <= 1.0))
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
            /* training: dropout on the way up (Xl is this layer's output) */
            if (drop_p > 0.0)
                for (size_t e = 0; e < seq_out; ++e) Xl[e] *= dropout_factor(drop_p, seed, call, l, e);
        }
    }
    memcpy(y, Y, sizeof(double) * seq_out);
    free(h); free(c); free(pre); free(Yl); free(Xl);
    return 0;
}

/* Gradients of the forward pass above (every row has all T steps).
 *   dy   [T][B][D*H] gradient of y;  dh_n, dc_n [L*D][B][H] or NULL (zeros)
 * Outputs (each may be NULL when not wanted):
 *   dx   [T][B][I];  dh0, dc0 [L*D][B][H];
 *   dparams: same order and shapes as params (W_ih, W_hh[, b_ih, b_hh]),
 *            overwritten (not accumulated into)
 * drop_p, seed, call: the dropout of the training forward (drop_p = 0: none).
 * lengths: NULL or per-row lengths as in oracle_lstm_forward_lengths.  At a
 * padded step the forward left h and c alone and output 0, so there the
 * pre-activation gradients are 0, and the cell-state gradient and the
 * gradient of h pass on to the step before unchanged.
 * The forward is recomputed here; its per-step activations are kept. */
int oracle_lstm_backward(int T, int B, int I, int H, int L, int D,
                         const double *x, const int *lengths, const double *h0, const double *c0,
                         const double *const *params, int has_bias,
                         double drop_p, uint64_t seed, uint64_t call,
                         const double *dy, const double *dh_n, const double *dc_n,
                         double *dx, double *dh0, double *dc0, double *const *dparams)
{
    if (T < 1 || B < 1 || I < 1 || H < 1 || L < 1 || (D != 1 && D != 2) || !x || !params || !dy ||
        !(drop_p >= 0.0 && drop_p <= 1.0))
        return -1;
    if (lengths)
        for (int b = 0; b < B; ++b)
            if (lengths[b] < 1 || lengths[b] > T) return -1;
    const int per = has_bias ? 4 : 2;
    const int G = 4 * H;
    const size_t BH = (size_t)B * H, TBH = (size_t)T * BH;
    const int win = I > D * H ? I : D * H;
    /* saved forward activations, per (layer, direction): gates i,f,g,o and c, h at every t */
    const size_t nld = (size_t)L * D;
    double *gi = malloc(sizeof(double) * nld * TBH), *gf = malloc(sizeof(double) * nld * TBH);
    double *gg = malloc(sizeof(double) * nld * TBH), *go = malloc(sizeof(double) * nld * TBH);
    double *cs = malloc(sizeof(double) * nld * TBH), *hs = malloc(sizeof(double) * nld * TBH);
    double *seq = malloc(sizeof(double) * (size_t)(L + 1) * T * B * win);  /* input of each layer */
    double *dY = malloc(sizeof(double) * (size_t)T * B * win), *dX = malloc(sizeof(double) * (size_t)T * B * win);
    double *dz = malloc(sizeof(double) * (size_t)B * G);
    double *dh = malloc(sizeof(double) * BH), *dc = malloc(sizeof(double) * BH), *dhn = malloc(sizeof(double) * BH);
    double *h = malloc(sizeof(double) * BH), *c = malloc(sizeof(double) * BH);
    int rc = -2;
    if (!gi || !gf || !gg || !go || !cs || !hs || !seq || !dY || !dX || !dz || !dh || !dc || !dhn || !h || !c)
        goto out;
    /* ---- forward, keeping activations */
    for (size_t e = 0; e < (size_t)T * B * I; ++e) seq[e] = x[e];
    for (int l = 0; l < L; ++l) {
        const int in_w = l == 0 ? I : D * H;
        const double *in_seq = seq + (size_t)l * T * B * win;
        double *out_seq = seq + (size_t)(l + 1) * T * B * win;
        for (int d = 0; d < D; ++d) {
            const double *const *p = params + (size_t)(l * D + d) * per;
            const size_t st = (size_t)(l * D + d) * BH, ld = (size_t)(l * D + d) * TBH;
            for (size_t e = 0; e < BH; ++e) {
                h[e] = (h0 != NULL) ? h0[st + e] : 0.0;
                c[e] = (c0 != NULL) ? c0[st + e] : 0.0;
            }
            for (int s = 0; s < T; ++s) {
                const int t = d == 0 ? s : T - 1 - s;
                for (int b = 0; b < B; ++b) {
                    if (PADDED(t, b)) {  /* the state stays; the output is 0 */
                        for (int j = 0; j < H; ++j) {
                            const size_t e = ld + (size_t)t * BH + (size_t)b * H + j;
                            gi[e] = gf[e] = gg[e] = go[e] = 0.0;
                            cs[e] = c[(size_t)b * H + j];
                            hs[e] = h[(size_t)b * H + j];
                            out_seq[((size_t)t * B + b) * (D * H) + (size_t)d * H + j] = 0.0;
                        }
                        continue;
                    }
                    const double *xt = in_seq + ((size_t)t * B + b) * in_w;
                    double pre[4];
                    for (int j = 0; j < H; ++j) {
                        for (int q = 0; q < 4; ++q) {
                            const int r = q * H + j;
                            double acc = has_bias ? p[2][r] + p[3][r] : 0.0;
                            for (int k = 0; k < in_w; ++k) acc += p[0][(size_t)r * in_w + k] * xt[k];
                            for (int k = 0; k < H; ++k) acc += p[1][(size_t)r * H + k] * h[(size_t)b * H + k];
                            pre[q] = acc;
                        }
                        const size_t e = ld + (size_t)t * BH + (size_t)b * H + j;
                        gi[e] = sigmoid(pre[0]);
                        gf[e] = sigmoid(pre[1]);
                        gg[e] = tanh(pre[2]);
                        go[e] = sigmoid(pre[3]);
                    }
                    for (int j = 0; j < H; ++j) {
                        const size_t e = ld + (size_t)t * BH + (size_t)b * H + j;
                        cs[e] = gf[e] * c[(size_t)b * H + j] + gi[e] * gg[e];
                        hs[e] = go[e] * tanh(cs[e]);
                    }
                    for (int j = 0; j < H; ++j) {
                        const size_t e = ld + (size_t)t * BH + (size_t)b * H + j;
                        c[(size_t)b * H + j] = cs[e];
                        h[(size_t)b * H + j] = hs[e];
                        /* the next layer's input, through the training dropout */
                        const size_t oe = ((size_t)t * B + b) * (D * H) + (size_t)d * H + j;
                        out_seq[oe] = l + 1 < L ? hs[e] * dropout_factor(drop_p, seed, call, l, oe) : hs[e];
                    }
                }
            }
        }
    }
    /* ---- backward, top layer first */
    for (size_t e = 0; e < (size_t)T * B * D * H; ++e) dY[e] = dy[e];
    for (int l = L - 1; l >= 0; --l) {
        const int in_w = l == 0 ? I : D * H;
        const double *in_seq = seq + (size_t)l * T * B * win;
        memset(dX, 0, sizeof(double) * (size_t)T * B * in_w);
        for (int d = 0; d < D; ++d) {
            const double *const *p = params + (size_t)(l * D + d) * per;
            double *const *dp = dparams ? dparams + (size_t)(l * D + d) * per : NULL;
            const size_t st = (size_t)(l * D + d) * BH, ld = (size_t)(l * D + d) * TBH;
            if (dp) {
                memset(dp[0], 0, sizeof(double) * (size_t)G * in_w);
                memset(dp[1], 0, sizeof(double) * (size_t)G * H);
                if (has_bias) {
                    memset(dp[2], 0, sizeof(double) * G);
                    memset(dp[3], 0, sizeof(double) * G);
                }
            }
            /* gradients arriving from after the last step: those of h_n, c_n */
            for (size_t e = 0; e < BH; ++e) {
                dhn[e] = dh_n ? dh_n[st + e] : 0.0;
                dc[e] = dc_n ? dc_n[st + e] : 0.0;
            }
            /* walk the scan backwards: s = T-1 is the step the scan took last */
            for (int s = T - 1; s >= 0; --s) {
                const int t = d == 0 ? s : T - 1 - s;
                const int tp = d == 0 ? t - 1 : t + 1; /* time of the scan's previous step */
                for (int b = 0; b < B; ++b) {
                    if (PADDED(t, b)) {  /* no gate took part: dc (and dh, below) pass on unchanged */
                        for (int r = 0; r < G; ++r) dz[(size_t)b * G + r] = 0.0;
                        continue;
                    }
                    for (int j = 0; j < H; ++j) {
                        const size_t e = ld + (size_t)t * BH + (size_t)b * H + j;
                        const size_t eb = (size_t)b * H + j;
                        /* h_t feeds y_t and the next step's products */
                        const size_t ye = ((size_t)t * B + b) * (D * H) + (size_t)d * H + j;
                        const double dht = dY[ye] + dhn[eb];
                        const double tc = tanh(cs[e]);
                        const double cprev = s == 0 ? (c0 ? c0[st + eb] : 0.0) : cs[ld + (size_t)tp * BH + eb];
                        /* h = o tanh(c);  c = f c_prev + i g */
                        const double dct = dc[eb] + dht * go[e] * (1.0 - tc * tc);
                        dz[(size_t)b * G + 3 * H + j] = dht * tc * go[e] * (1.0 - go[e]);
                        dz[(size_t)b * G + j] = dct * gg[e] * gi[e] * (1.0 - gi[e]);
                        dz[(size_t)b * G + 2 * H + j] = dct * gi[e] * (1.0 - gg[e] * gg[e]);
                        dz[(size_t)b * G + H + j] = dct * cprev * gf[e] * (1.0 - gf[e]);
                        dc[eb] = dct * gf[e];  /* to c_prev */
                    }
                }
                /* the pre-activations are W_ih x_t + W_hh h_prev + b_ih + b_hh */
                for (int b = 0; b < B; ++b) {
                    const double *xt = in_seq + ((size_t)t * B + b) * in_w;
                    for (int k = 0; k < H; ++k) {
                        const double hprev = s == 0 ? (h0 ? h0[st + (size_t)b * H + k] : 0.0)
                                                    : hs[ld + (size_t)tp * BH + (size_t)b * H + k];
                        h[(size_t)b * H + k] = hprev;
                    }
                    for (int k = 0; k < H; ++k) {
                        double acc = 0.0;
                        for (int r = 0; r < G; ++r) acc += dz[(size_t)b * G + r] * p[1][(size_t)r * H + k];
                        /* a padded step's h was its predecessor's: its gradient passes through */
                        dh[(size_t)b * H + k] = PADDED(t, b) ? dhn[(size_t)b * H + k] : acc;
                    }
                    for (int k = 0; k < in_w; ++k) {
                        double acc = 0.0;
                        for (int r = 0; r < G; ++r) acc += dz[(size_t)b * G + r] * p[0][(size_t)r * in_w + k];
                        dX[((size_t)t * B + b) * in_w + k] += acc;
                    }
                    if (dp) {
                        for (int r = 0; r < G; ++r) {
                            const double z = dz[(size_t)b * G + r];
                            for (int k = 0; k < in_w; ++k) dp[0][(size_t)r * in_w + k] += z * xt[k];
                            for (int k = 0; k < H; ++k) dp[1][(size_t)r * H + k] += z * h[(size_t)b * H + k];
                            if (has_bias) {
                                dp[2][r] += z;
                                dp[3][r] += z;
                            }
                        }
                    }
                }
                for (size_t e = 0; e < BH; ++e) dhn[e] = dh[e];
            }
            if (dh0) memcpy(dh0 + st, dhn, sizeof(double) * BH);
            if (dc0) memcpy(dc0 + st, dc, sizeof(double) * BH);
        }
        /* the layer below receives the gradient of its output sequence,
         * through the dropout factor that output was sent up with */
        for (size_t e = 0; e < (size_t)T * B * in_w; ++e)
            dY[e] = l > 0 ? dX[e] * dropout_factor(drop_p, seed, call, l - 1, e) : dX[e];
    }
    if (dx) memcpy(dx, dY, sizeof(double) * (size_t)T * B * I);
    rc = 0;
out:
    free(gi); free(gf); free(gg); free(go); free(cs); free(hs); free(seq); free(dY); free(dX);
    free(dz); free(dh); free(dc); free(dhn); free(h); free(c);
    return rc;
}

int oracle_lstm_forward_lengths(int T, int B, int I, int H, int L, int D,
                                const double *x, const int *lengths,
                                const double *h0, const double *c0,
                                const double *const *params, int has_bias,
                                double *y, double *h_n, double *c_n, int nthreads)
{
    return forward_core(T, B, I, H, L, D, x, lengths, h0, c0, params, has_bias, 0.0, 0, 0,
                        y, h_n, c_n, nthreads);
}

/* Every row has all T steps. */
int oracle_lstm_forward(int T, int B, int I, int H, int L, int D,
                        const double *x, const double *h0, const double *c0,
                        const double *const *params, int has_bias,
                        double *y, double *h_n, double *c_n, int nthreads)
{
    return forward_core(T, B, I, H, L, D, x, NULL, h0, c0, params, has_bias, 0.0, 0, 0,
                        y, h_n, c_n, nthreads);
}

/* Training forward: dropout with probability p between layers; lengths as
 * for oracle_lstm_forward_lengths, or NULL. */
int oracle_lstm_forward_dropout(int T, int B, int I, int H, int L, int D,
                                const double *x, const int *lengths, const double *h0, const double *c0,
                                const double *const *params, int has_bias,
                                double p, uint64_t seed, uint64_t call,
                                double *y, double *h_n, double *c_n, int nthreads)
{
    return forward_core(T, B, I, H, L, D, x, lengths, h0, c0, params, has_bias, p, seed, call,
                        y, h_n, c_n, nthreads);
}

/* Forward pass of the other recurrent modes: mode 1 GRU, 2 RNN_TANH, 3
 * RNN_RELU.  Parameters per (layer, direction): W_ih [NG*H][in_l],
 * W_hh [NG*H][H] (and b_ih, b_hh [NG*H] when has_bias), NG = 3 for the GRU
 * and 1 for the RNNs.  h0, h_n [L*D][B][H] as for the LSTM; no cell state.
 * lengths: NULL or per-row lengths with the LSTM's reading (a padded step
 * leaves h alone and outputs 0).
 * Returns 0, -1 on a bad argument, -2 if memory runs out. */
int oracle_rnn_forward(int mode, int T, int B, int I, int H, int L, int D,
                       const double *x, const int *lengths, const double *h0, const double *const *params,
                       int has_bias, double *y, double *h_n, int nthreads)
{
    if (mode < 1 || mode > 3 || T < 1 || B < 1 || I < 1 || H < 1 || L < 1 || (D != 1 && D != 2) ||
        !x || !params || !y)
        return -1;
    if (lengths)
        for (int b = 0; b < B; ++b)
            if (lengths[b] < 1 || lengths[b] > T) return -1;
    if (nthreads < 1) nthreads = 1;
    const int per = has_bias ? 4 : 2;
    const int NG = mode == 1 ? 3 : 1, R = NG * H;
    const size_t nseq = (size_t)T * B * D * H;
    double *state = malloc(sizeof(double) * (size_t)B * H);
    double *gin = malloc(sizeof(double) * (size_t)B * R), *ghid = malloc(sizeof(double) * (size_t)B * R);
    double *cur = malloc(sizeof(double) * nseq), *below = malloc(sizeof(double) * nseq);
    if (!state || !gin || !ghid || !cur || !below) {
        free(state); free(gin); free(ghid); free(cur); free(below);
        return -2;
    }
    const double *src = x;
    int width = I;
    for (int l = 0; l < L; ++l) {
        memset(cur, 0, sizeof(double) * nseq);
        for (int d = 0; d < D; ++d) {
            const double *const *w = params + (size_t)(l * D + d) * per;
            const size_t base = (size_t)(l * D + d) * B * H;
            for (size_t q = 0; q < (size_t)B * H; ++q) state[q] = h0 ? h0[base + q] : 0.0;
            for (int s = 0; s < T; ++s) {
                const int t = d == 0 ? s : T - 1 - s;
                /* the input and the hidden contributions of every gate row, kept apart */
#pragma omp parallel for collapse(2) num_threads(nthreads) if (nthreads > 1)
                for (int b = 0; b < B; ++b) {
                    for (int r = 0; r < R; ++r) {
                        const double *xv = src + ((size_t)t * B + b) * width;
                        double a = has_bias ? w[2][r] : 0.0, c = has_bias ? w[3][r] : 0.0;
                        for (int k = 0; k < width; ++k) a += w[0][(size_t)r * width + k] * xv[k];
                        for (int k = 0; k < H; ++k) c += w[1][(size_t)r * H + k] * state[(size_t)b * H + k];
                        gin[(size_t)b * R + r] = a;
                        ghid[(size_t)b * R + r] = c;
                    }
                }
                for (int b = 0; b < B; ++b) {
                    if (PADDED(t, b)) continue;  /* h stays, y stays 0 */
                    for (int j = 0; j < H; ++j) {
                        const double *gi = gin + (size_t)b * R, *gh = ghid + (size_t)b * R;
                        double hv;
                        if (mode == 1) {
                            const double rg = sigmoid(gi[j] + gh[j]);
                            const double zg = sigmoid(gi[H + j] + gh[H + j]);
                            const double ng = tanh(gi[2 * H + j] + rg * gh[2 * H + j]);
                            hv = (1.0 - zg) * ng + zg * state[(size_t)b * H + j];
                        } else {
                            const double v = gi[j] + gh[j];
                            hv = mode == 2 ? tanh(v) : (v > 0.0 ? v : 0.0);
                        }
                        cur[((size_t)t * B + b) * (D * H) + (size_t)d * H + j] = hv;
                    }
                    /* every gate row of row b has read the old state: replace it */
                    for (int j = 0; j < H; ++j)
                        state[(size_t)b * H + j] = cur[((size_t)t * B + b) * (D * H) + (size_t)d * H + j];
                }
            }
            if (h_n) memcpy(h_n + base, state, sizeof(double) * (size_t)B * H);
        }
        /* the layer above reads this layer's output sequence */
        double *swap = below; below = cur; cur = swap;
        src = below;
        width = D * H;
    }
    memcpy(y, below, sizeof(double) * nseq);
    free(state); free(gin); free(ghid); free(cur); free(below);
    return 0;
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
