/*
 * lstm.h -- C ABI of the MI355X (gfx950) LSTM forward library liblstm_amd.so.
 *
 * The operation: a multi-layer, optionally bidirectional LSTM forward pass.
 * Per layer, direction and time step (warp-nn "Long Short-Term Memory (LSTM)",
 * the equation block under the class signature):
 *     i = sigma(W_ii x + b_ii + W_hi h + b_hi)   f = sigma(... f rows ...)
 *     g = tanh (W_ig x + b_ig + W_hg h + b_hg)   o = sigma(... o rows ...)
 *     c' = f*c + i*g                             h' = o*tanh(c')
 * Layer k > 0 reads the D*H-wide output of layer k-1 (same page, the symbol
 * list); the reverse direction scans from the last element to the first with
 * its own parameters and its hidden states are concatenated after the
 * forward ones (same page, the paragraph on bidirectional).  Inputs, outputs
 * and return values follow the op signature traced on "Complete Trace:
 * nn.LSTM" (Step 3, lstm.input -> (output, h_n, c_n)) and warp-nn __call__.
 *
 * Conventions
 *   - All tensors are dense, row-major and time-major ([T, B, .]); batch-first
 *     callers transpose before the call.
 *   - dtype LSTM_F32: x, weights, biases, h0, y, h_n are float32.
 *     dtype LSTM_BF16: the same tensors are bfloat16; arithmetic accumulates in
 *     float32, the cell state c0 / c_n stays float32 in both modes, and the
 *     hidden state is rounded to bfloat16 (nearest-even) where it is stored.
 *   - Every tensor pointer is device memory on the current HIP device, owned
 *     by the caller.  The library allocates no device memory; all scratch
 *     lives in the caller's workspace (lstm_forward_static: in the library's
 *     own file-scope device array).
 *   - Weight pointer order (warp-nn "Learnable parameters" table, flattened
 *     layer by layer as "Complete Trace: nn.LSTM" Step 1 flattens them):
 *         for l in 0..L-1, for d in 0..D-1 (forward, then reverse):
 *             W_ih [4H, in_l]   in_0 = input_size, in_l = D*H for l > 0
 *             W_hh [4H, H]
 *             b_ih [4H]         only when has_bias
 *             b_hh [4H]         only when has_bias
 *     with the 4H rows in gate blocks [i; f; g; o] of H rows each.  Both
 *     biases are added.  Reading weights the caller has not written is the
 *     caller's undefined behaviour, as on the warp-nn page
 *     (initialize_parameters=False).
 *   - State index order of h0, c0, h_n, c_n [L*D, B, H]: l*D + d.  The
 *     reverse direction's final state is the one after consuming t = 0.
 *
 * Errors: every call returns an lstm_status.  Argument checks run on the host
 * before anything is enqueued; a failed check writes nothing.  Kernel-side
 * failures are asynchronous and are read back with lstm_device_status.
 * Nothing is printed and no C++ exception crosses this interface.
 */
#ifndef LSTM_AMD_LSTM_H
#define LSTM_AMD_LSTM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lstm_plan lstm_plan; /* opaque, immutable shape description */

typedef enum { LSTM_F32 = 0, LSTM_BF16 = 1 } lstm_dtype;

/* Recurrent modes.  The trace page's RNNBase ("Complete Trace: nn.LSTM",
 * Step 1) takes a mode among LSTM, GRU, RNN_TANH and RNN_RELU, and gives the
 * equations of the LSTM only; the others follow the definitions of the
 * framework whose RNNBase that page reproduces.  With gi = W_ih x_t + b_ih
 * and gh = W_hh h + b_hh in H-row blocks:
 *   GRU (blocks r, z, n):  r = sigma(gi_r + gh_r), z = sigma(gi_z + gh_z),
 *                          n = tanh(gi_n + r * gh_n), h' = (1 - z) n + z h
 *   RNN_TANH: h' = tanh(gi + gh);   RNN_RELU: h' = max(0, gi + gh)
 * W_ih, W_hh and the biases have 3H (GRU) or H (RNN) rows instead of 4H;
 * there is no cell state. */
typedef enum { LSTM_MODE_LSTM = 0, LSTM_MODE_GRU = 1, LSTM_MODE_RNN_TANH = 2, LSTM_MODE_RNN_RELU = 3 } lstm_mode;

typedef enum {
    LSTM_OK = 0,
    LSTM_ERR_ARG = -1,         /* NULL/negative argument, num_layers < 1, h0 without c0 */
    LSTM_ERR_SHAPE = -2,       /* T < 1, B < 1, layers/bidir differ from the plan, size overflow */
    LSTM_ERR_DTYPE = -3,       /* unknown dtype */
    LSTM_ERR_DEVICE = -4,      /* a pointer is not device memory of the current device, or no device */
    LSTM_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than lstm_workspace_size */
    LSTM_ERR_LAUNCH = -6,      /* a kernel launch was refused by the runtime */
    LSTM_ERR_UNSUPPORTED = -7, /* option value not supported */
    LSTM_ERR_DEVICE_TIMEOUT = -8 /* lstm_device_status: a step barrier gave up waiting */
} lstm_status;

/* Recurrent-phase execution modes (lstm_set_option LSTM_OPT_RECURRENCE). */
typedef enum {
    LSTM_REC_AUTO = 0,       /* persistent when the plan's W_hh slices fit on chip, else per step as a
                                GEMM when rows are 16-byte aligned, else per step with the tile kernel */
    LSTM_REC_STEP = 1,       /* one launch of the tile kernel per time step (no cross-workgroup waits) */
    LSTM_REC_PERSISTENT = 2, /* one cooperative launch per layer; LSTM_ERR_UNSUPPORTED if it does not fit */
    LSTM_REC_GEMM = 3        /* one launch per time step of a GEMM-shaped kernel (64 rows x 32 units per
                                workgroup, cell update fused); needs H*sizeof(dtype) a multiple of 16,
                                16-byte aligned y, h0 and W_hh, else LSTM_ERR_UNSUPPORTED */
} lstm_recurrence;

typedef enum {
    LSTM_OPT_RECURRENCE = 1, /* value: lstm_recurrence */
    LSTM_OPT_REC_TILE = 2,   /* value: 0 = automatic, else 100*WK + 10*MTW + NT (see lstm_describe) */
    LSTM_OPT_TIMING = 3,     /* value 1: record HIP events around each phase (see lstm_read_timing) */
    LSTM_OPT_PARTIAL_BUFFERS = 4, /* 1 (default) or 2 LDS partial-sum buffers in the recurrent kernel */
    LSTM_OPT_POLL_SLEEP = 5, /* 0..1000: back-off (units of 64 clocks) between re-reads of h words */
    /* 6: reserved (no longer accepted) */
    LSTM_OPT_TEAM_ROWS = 7,  /* 0 (default): batch rows per team as the tile holds; n > 0: at most n */
    LSTM_OPT_PROJ_TILE = 8,  /* projection GEMM: 0 automatic (7 where the 256x256 direct-to-LDS tiles
                                apply), 1 128x128, 2 256x256, 3 256x256 direct-to-LDS,
                                4 / 5 256x256 direct-to-LDS through a ring of 4 / 5 stages, 6 256x128
                                through a ring of 3 stages (two workgroups per CU), 7 as 3 with the next
                                stage's loads interleaved with the products */
    LSTM_OPT_READ_PACE = 9,  /* 0..100000 ns (default by schedule: 300 to 450 for teams across XCDs, 0 on
                                one XCD): delay between a workgroup
                                finishing step t (its h_t published) and its first read of the other
                                workgroups' h_t; 0 reads as soon as the step ends. A read that reaches
                                memory before the data costs a retry round trip; results do not depend
                                on it */
    LSTM_OPT_LAYER_PIPE = 10, /* 1 (default): a unidirectional LSTM stack of 2..4 layers in the time-major
                                layout runs every layer in one persistent launch (the layer wavefront: layer
                                l consumes layer l-1's h_t as it is produced, two workgroups per CU) when its
                                tiles fit (H and the input width at most 128 fp32 / 256 bf16 values per wave
                                and whole 16-byte rows) and all its workgroups are co-resident; 2: the same,
                                with a two-layer stack's layers paired in 512-thread workgroups that step
                                in lockstep (layer 1 two steps behind; at most 8 units per workgroup);
                                0: layer by layer.  Not used with per-row lengths or in training. Changes
                                lstm_workspace_size. */
    LSTM_OPT_FUSE_INPUT = 11, /* 1 (default): a layer whose recurrence runs as one persistent launch and
                                whose W_ih share fits in registers computes x_t W_ih^T + b_ih + b_hh inside
                                that launch (no projection GEMM, G unused); 0: always hoist the projection */
    LSTM_OPT_SMALL_BATCH = 13, /* 1 (default): an LSTM layer with B <= 16 whose W_hh fits the registers of
                                one XCD's 32 CUs (H <= 1024 bf16 / 512 fp32, whole 16-byte rows) runs each
                                direction's recurrence on one XCD, after a hoisted projection; 0: the
                                general recurrence (time-major inference only, as the wavefront) */
    LSTM_OPT_RESIDENT = 14,    /* 1 (default): a bf16 LSTM layer whose W_hh is too large for the per-layer
                                persistent recurrence (H one of 256, 512, 1024, 1536, 2048, and
                                ceil(B/128)*D*H/16 workgroups fitting the chip at once) runs its recurrence
                                in one launch that holds W_hh once across the chip and exchanges h through
                                y; 2: whenever the shape allows it; 0: never (one launch per step).
                                Time-major inference only, without per-row lengths */
    LSTM_OPT_BATCH_FIRST = 12 /* 0 (default): x is [T, B, input_size] and y is [T, B, D*H]; 1: x is
                                [B, T, input_size] and y is [B, T, D*H] ("batch_first" of the trace page's
                                op signature, Step 3).  h0, c0, h_n, c_n stay [L*D, B, H].  A layout
                                option: unlike the others it changes what the pointers mean */
} lstm_option;

/* Accumulated per-phase device time of the calls made since the last reset
 * (LSTM_OPT_TIMING).  A "launch" is one kernel launch of that phase: one
 * projection GEMM per layer; one recurrent launch per layer when persistent,
 * T per layer when stepping.  Backward phases (lstm_backward): a "launch" of
 * the recurrence is one backward step (its product and cell launches; the
 * events bracket a layer's whole loop of T steps); one of the gradient
 * products is one weight or input gradient (GEMM and slab sum). */
typedef struct {
    double proj_ms;     /* input-projection GEMMs */
    double rec_ms;      /* recurrent kernels */
    int calls;          /* lstm_forward / lstm_forward_train calls timed */
    int proj_launches;
    int rec_launches;
    double bwd_rec_ms;  /* backward recurrence: products dz_t W_hh and cell updates */
    double bwd_gemm_ms; /* backward weight- and input-gradient products */
    int bwd_calls;      /* lstm_backward calls timed */
    int bwd_rec_launches;
    int bwd_gemm_launches;
} lstm_timing;

/* Create a plan.  input_size, hidden_size >= 1; num_layers >= 1 (warp-nn
 * "Raises": fewer than one layer is an error); bidirectional and has_bias are
 * 0 or 1.  Touches no device.  *out receives the handle (NULL on error). */
lstm_status lstm_create(lstm_plan **out, int input_size, int hidden_size, int num_layers,
                        int bidirectional, int has_bias, int dtype);

/* lstm_create for any lstm_mode (lstm_create is mode LSTM_MODE_LSTM); a mode
 * outside the enum is LSTM_ERR_ARG.  For the GRU and the RNNs, lstm_forward
 * takes h0 alone (c0 and c_n must be NULL, else LSTM_ERR_ARG).  Where an LSTM
 * of the same shape gets a persistent recurrence, they run on it with their
 * gate blocks copied into the workspace padded to four; otherwise (or with
 * LSTM_REC_STEP / LSTM_REC_GEMM) one projection GEMM and T recurrent-step
 * launches per layer, which need hidden_size * element size to be a multiple
 * of 16 bytes and 16-byte aligned x, y, h0 and weights
 * (LSTM_ERR_UNSUPPORTED otherwise).  lstm_forward_lengths takes them on either
 * path: a padded step keeps the row's h and writes zeros to y, as for the LSTM.
 * The training entry points and their size queries are LSTM_ERR_UNSUPPORTED. */
lstm_status lstm_create_mode(lstm_plan **out, int mode, int input_size, int hidden_size, int num_layers,
                             int bidirectional, int has_bias, int dtype);

/* Release a plan (NULL is ignored). */
void lstm_destroy(lstm_plan *plan);

/* Set an execution option.  Options change how the forward is scheduled, not
 * what it computes (LSTM_OPT_BATCH_FIRST alone changes the layout of x and y). */
lstm_status lstm_set_option(lstm_plan *plan, int option, int value);

/* Bytes of device workspace lstm_forward needs for sequence length T and batch
 * B (intermediate layer outputs, the hoisted input projection, cell-state and
 * synchronisation words).  Touches no device.  The caller queries the size,
 * allocates the workspace and passes it to the forward call, the sequence the
 * trace page "Complete Trace: nn.LSTM" (Step 5, the fused-library path) shows
 * for its workspace. */
lstm_status lstm_workspace_size(const lstm_plan *plan, int T, int B, size_t *bytes);

/* Enqueue the forward pass on `stream` (a hipStream_t; NULL = default stream).
 *   x        [T, B, input_size]            dtype
 *   h0       [L*D, B, H] dtype, or NULL    NULL means zeros; h0 and c0 are
 *   c0       [L*D, B, H] float32, or NULL  given together or not at all
 *   weights  host array of L*D*(has_bias ? 4 : 2) device pointers, order above
 *   T, B     sequence length and batch size, both >= 1
 *   layers, bidir  must equal the plan's (checked, not trusted)
 *   y        [T, B, D*H]                   dtype, written
 *   h_n      [L*D, B, H] dtype, or NULL    written if not NULL
 *   c_n      [L*D, B, H] float32, or NULL  written if not NULL
 *   workspace, workspace_bytes  device scratch of at least lstm_workspace_size
 *   bytes; its contents are overwritten; it must not be shared by calls that
 *   can run concurrently.
 * Returns after enqueueing; results are ready when the stream reaches them.
 * Inputs must not alias outputs or the workspace. */
lstm_status lstm_forward(lstm_plan *plan, const void *x, const void *h0, const float *c0,
                         const void *const *weights, int T, int B, int layers, int bidir,
                         void *y, void *h_n, float *c_n, void *workspace,
                         size_t workspace_bytes, void *stream);

/* lstm_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture into a graph, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a file-scope device
 * array of LSTM_STATIC_WORKSPACE_BYTES inside the library: one copy on each
 * device the library runs on, held until the process ends, its address looked
 * up once per device.  The call allocates nothing (no hipMalloc, no allocating
 * library routine).
 *   x .. c_n, stream  as lstm_forward
 *   device_status     device memory for one unsigned, or NULL: after the
 *                     forward, a one-thread kernel on `stream` copies the
 *                     kernel status word there (0: every step barrier
 *                     completed; non-zero: a wait gave up and the outputs are
 *                     invalid), what lstm_device_status reads for lstm_forward
 * Errors as lstm_forward; a (T, B) whose lstm_workspace_size exceeds
 * LSTM_STATIC_WORKSPACE_BYTES is LSTM_ERR_WORKSPACE, with nothing enqueued.
 * Every call on one device shares that device's array, and each call
 * overwrites it (the synchronisation words are cleared at the start of each
 * call, on its stream): calls that can overlap on one device -- on different
 * streams, or from several threads -- race and must be serialised by the
 * caller. */
#define LSTM_STATIC_WORKSPACE_BYTES ((size_t)96 << 20)
lstm_status lstm_forward_static(lstm_plan *plan, const void *x, const void *h0, const float *c0,
                                const void *const *weights, int T, int B, int layers, int bidir, void *y,
                                void *h_n, float *c_n, unsigned *device_status, void *stream);

/* Variable-length batches: the same forward with a sequence length per
 * batch row on the padded [T, B, .] layout.  The trace page "Complete Trace:
 * nn.LSTM" (Step 3) lists a packed-sequence overload beside the padded one,
 * and the MXNet blog "LSTM Forward Computation" ("Sequence Buckets") pads
 * sequences of different lengths and ignores the padded elements.
 *   lengths  HOST array of B int32 values in 1..T (read before the call
 *            returns; the library copies it into the workspace).  Row b takes
 *            part only in the steps t < lengths[b]: its state is left as it is
 *            at the other steps and y[t, b, :] = 0 there; h_n and c_n are the
 *            state after the row's last valid step, and the reverse direction
 *            starts at t = lengths[b] - 1 from h0/c0.  (A packed batch_sizes
 *            tensor of rows sorted by length gives lengths[b] = the number of
 *            steps t with batch_sizes[t] > b.)
 * Every other argument, the outputs and the errors are those of lstm_forward;
 * a NULL lengths or a value outside 1..T is LSTM_ERR_ARG and nothing is
 * enqueued.  The layer pipeline (LSTM_OPT_LAYER_PIPE) is not used here. */
lstm_status lstm_forward_lengths(lstm_plan *plan, const void *x, const int *lengths, const void *h0,
                                 const float *c0, const void *const *weights, int T, int B, int layers,
                                 int bidir, void *y, void *h_n, float *c_n, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* Packed sequences, the other overload the trace page "Complete Trace:
 * nn.LSTM" (Step 3) lists: x is [N, input_size] (dtype), the rows of step t
 * being rows o_t .. o_t + batch_sizes[t] - 1 with o_t = the sum of the
 * earlier batch_sizes, one per sequence still running at t; sequences are in
 * order of non-increasing length, so batch_sizes is non-increasing.
 *   batch_sizes  HOST array of T int32 values, batch_sizes[0] = B (the
 *                number of sequences) >= batch_sizes[1] >= ... >= 1;
 *                N = their sum.  Read before the call returns.
 *   y            [N, D*H] dtype, packed like x
 *   h_n, c_n     [L*D, B, H] as lstm_forward, rows in the packed sequence
 *                order (h0 and c0 likewise)
 *   workspace    at least lstm_packed_workspace_size bytes
 * The result equals lstm_forward_lengths on the padded [T, B, .] layout with
 * lengths[b] = the number of steps t with batch_sizes[t] > b: the rows are
 * gathered into a zero-padded buffer in the workspace, that forward runs, and
 * y is scattered back.  A NULL batch_sizes, an increasing or a non-positive
 * entry is LSTM_ERR_ARG; a plan with LSTM_OPT_BATCH_FIRST set is
 * LSTM_ERR_UNSUPPORTED; other errors as lstm_forward_lengths. */
lstm_status lstm_packed_workspace_size(const lstm_plan *plan, const int *batch_sizes, int T, size_t *bytes);
lstm_status lstm_forward_packed(lstm_plan *plan, const void *x, const int *batch_sizes, int T, const void *h0,
                                const float *c0, const void *const *weights, int layers, int bidir, void *y,
                                void *h_n, float *c_n, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ training
 * Backward pass (backpropagation through time).  The trace page "Complete
 * Trace: nn.LSTM" ("cuDNN Backward") computes the gradients of the input, of
 * the initial states and of the weights from the gradients of (output, h_n,
 * c_n) and a reserve of activations saved by the forward; the pulsatrix
 * "LSTMModule" reference describes the backpropagation through time across
 * the four gates and the cell carry.  Both layouts (with LSTM_OPT_BATCH_FIRST
 * x, y, dy and dx are [B, T, .]); per-row lengths through the _lengths
 * variants; the LSTM mode only (others: LSTM_ERR_UNSUPPORTED). */

/* Training dropout between layers.  The trace page's Performance Notes apply
 * dropout to the input of every layer above the first, in training only
 * (lstm_forward never drops); its Step 3 op signature carries the
 * probability.  With probability prob in [0, 1] (0: none, the default),
 * element e of layer l's output ([T, B, D*H] flat, time-major) reaches layer
 * l + 1 as y * 1/(1 - prob) when kept and as 0 when dropped (all dropped when
 * prob = 1).  The draw is Philox4x64-10 (Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC 2011): the block with
 * counter (e / 4, l, call, 0) and key (seed, 0) gives four 64-bit words, and
 * word e % 4 keeps e when (word >> 11) * 2^-53 >= prob.  `call` is the index
 * used by the next lstm_forward_train; each successful call with dropout
 * advances it by one.  Set it before lstm_reserve_size (the reserve then also
 * holds each dropped layer input and its keep bytes) and keep it unchanged
 * between a lstm_forward_train and its lstm_backward.  prob outside [0, 1]
 * (or NaN) is LSTM_ERR_ARG. */
lstm_status lstm_set_dropout(lstm_plan *plan, double prob, unsigned long long seed, unsigned long long call);

/* Bytes of reserve lstm_forward_train fills for (T, B): per layer the gates
 * i, f, g, o and the cell state c of every step (fp32), and the outputs of
 * every layer but the top one (dtype); with dropout also, for every layer but
 * the top one, its output after dropout (dtype) and one keep byte per
 * element. */
lstm_status lstm_reserve_size(const lstm_plan *plan, int T, int B, size_t *bytes);

/* lstm_forward, and also fills `reserve` (device memory of at least
 * lstm_reserve_size bytes, caller-owned) for lstm_backward.  The layer
 * pipeline is not used.  Errors as lstm_forward; a NULL reserve is
 * LSTM_ERR_ARG, a short one LSTM_ERR_WORKSPACE. */
lstm_status lstm_forward_train(lstm_plan *plan, const void *x, const void *h0, const float *c0,
                               const void *const *weights, int T, int B, int layers, int bidir, void *y,
                               void *h_n, float *c_n, void *reserve, size_t reserve_bytes, void *workspace,
                               size_t workspace_bytes, void *stream);

/* lstm_forward_train over per-row lengths (B host values in 1..T, as for
 * lstm_forward_lengths): the reserve then also serves lstm_backward_lengths
 * with the same lengths.  NULL lengths or a length outside 1..T is
 * LSTM_ERR_ARG. */
lstm_status lstm_forward_train_lengths(lstm_plan *plan, const void *x, const int *lengths, const void *h0,
                                       const float *c0, const void *const *weights, int T, int B, int layers,
                                       int bidir, void *y, void *h_n, float *c_n, void *reserve,
                                       size_t reserve_bytes, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace lstm_backward needs for (T, B) (all fp32: the
 * pre-activation gradients of a layer and their transpose, transposed
 * operands, two output-gradient buffers, partial sums). */
lstm_status lstm_backward_workspace_size(const lstm_plan *plan, int T, int B, size_t *bytes);

/* Gradients of the forward that lstm_forward_train computed with the same x,
 * h0, c0, weights and reserve.
 *   y            [T, B, D*H] dtype, the output of that forward
 *   dy           [T, B, D*H] dtype, gradient of y
 *   dh_n         [L*D, B, H] dtype, or NULL (zeros)
 *   dc_n         [L*D, B, H] float32, or NULL (zeros)
 *   dx           [T, B, input_size] dtype, or NULL (not wanted)
 *   dh0, dc0     [L*D, B, H] (dtype / float32), or NULL
 *   dweights     host array of device pointers with the order and shapes of
 *                `weights` (dtype), overwritten (not accumulated into); both
 *                bias gradients equal the sum of the gate pre-activation
 *                gradients
 *   workspace    at least lstm_backward_workspace_size bytes
 * Products accumulate in fp32 (bf16 operands are widened exactly); results
 * are rounded to the output dtype once.  Errors as lstm_forward; a short
 * reserve or workspace is LSTM_ERR_WORKSPACE, and B * D * 5 * hidden_size * 4
 * bytes (one step's saved activations) of 2^31 or more LSTM_ERR_UNSUPPORTED.
 * When the recurrent products' tiles would leave CUs idle, each tile's
 * product is split between two workgroups that meet through the workspace;
 * lstm_device_status on this workspace then reports a wait that gave up
 * (flag 2; the outputs are invalid). */
lstm_status lstm_backward(lstm_plan *plan, const void *x, const void *h0, const float *c0,
                          const void *const *weights, const void *y, const void *dy, const void *dh_n,
                          const float *dc_n, const void *reserve, size_t reserve_bytes, int T, int B, int layers,
                          int bidir, void *dx, void *dh0, float *dc0, void *const *dweights, void *workspace,
                          size_t workspace_bytes, void *stream);

/* lstm_backward of a lstm_forward_train_lengths call, with the same lengths.
 * At a padded step (t >= length of the row) the forward left h and c alone
 * and output 0, so no gate gradient arises there and the gradients of h and
 * c pass on unchanged to the step before; dy at padded steps is ignored and
 * dx there is 0.  NULL lengths or a length outside 1..T is LSTM_ERR_ARG. */
lstm_status lstm_backward_lengths(lstm_plan *plan, const void *x, const int *lengths, const void *h0,
                                  const float *c0, const void *const *weights, const void *y, const void *dy,
                                  const void *dh_n, const float *dc_n, const void *reserve, size_t reserve_bytes,
                                  int T, int B, int layers, int bidir, void *dx, void *dh0, float *dc0,
                                  void *const *dweights, void *workspace, size_t workspace_bytes, void *stream);

/* Synchronise `stream` and read the kernel status word a previous
 * lstm_forward (or lstm_backward, with its own workspace) left in
 * `workspace`: *device_flags = 0 if every step barrier completed.  Returns LSTM_ERR_DEVICE_TIMEOUT when a flag is set (the outputs
 * of that call are then invalid). */
lstm_status lstm_device_status(const void *workspace, size_t workspace_bytes, void *stream,
                               unsigned *device_flags);

/* Wait for the events recorded by timed calls and return their totals; with
 * reset != 0 the totals restart from zero afterwards.  The timing state
 * belongs to the plan: time calls from one stream at a time. */
lstm_status lstm_read_timing(lstm_plan *plan, lstm_timing *out, int reset);

/* Write a one-line, human-readable description of the schedule lstm_forward
 * would use for (T, B) into buf (kernels, tile, workgroups, mode). */
lstm_status lstm_describe(const lstm_plan *plan, int T, int B, char *buf, size_t len);

/* Static text for a status code. */
const char *lstm_strerror(int status);

/* ABI version of this header (major*100 + minor). */
int lstm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LSTM_AMD_LSTM_H */
