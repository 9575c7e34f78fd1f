// kernels.h -- host-side interface of the gfx950 kernels (internal; the public
// ABI is include/lstm.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lstm.h"

namespace lstm_amd {

enum DType { DT_F32 = 0, DT_BF16 = 1 };

// G[m][d*N + n] = sum_k X[m][k] * W_d[n][k] + b_ih_d[n] + b_hh_d[n]
//   X   [M, K] with row stride ldx (elements), dtype
//   W_d [N, K] row-major, dtype; N = 4H; d = 0..D-1 (blockIdx.z)
//   G   [M, D*N] float32
//   kchunk > 0 splits K: blockIdx.z = d * nsplit + s, split s sums K range
//   [s*kchunk, min(K, (s+1)*kchunk)) into its own slab G + s*M*D*N (no bias);
//   kchunk is a multiple of 64.  W rows keep the stride K.
struct ProjArgs {
    const void *X;
    const void *W[2];
    const void *b_ih[2];
    const void *b_hh[2];
    float *G;
    int M, N, K, ldx, D;
    int kchunk;
};

// One layer of the recurrence for all directions and batch rows.
struct RecArgs {
    const void *whh[2];      // [4H, H] per direction, dtype
    const float *G;          // [T, B, D*4H] projection incl. both biases
    const void *h0;          // [D, B, H] dtype for this layer, or NULL (zeros)
    const float *c0;         // [D, B, H] or NULL
    void *Y;                 // [T, B, D*H] dtype, written
    void *hn;                // [D, B, H] dtype or NULL
    float *cn;               // [D, B, H] or NULL
    float *cstate;           // [D, B, H] carry between step launches
    float *hstate;           // [D, B, H] h carry between step launches (k_rec with lengths)
    const int *len;          // [B] valid steps per batch row, or NULL (all T)
    int bfirst;              // x, G, y rows are (b, t) = b*T + t instead of t*B + b
    float *acts;             // training: [T, B, D, 5, H] gates i, f, g, o and c of every step, or NULL
    unsigned long long *xbuf;  // h exchange: [2][D][NGB] regions of (ROWS/16)*kch*256 32-bit words (twice that when xwide)
    unsigned xpar;           // bit p: parity of the writes buffer p received before this launch
    int xwide;               // bf16: one value per exchange word (any h), else pairs (|h| < 2 only)
    unsigned *status;        // error word
    int T, B, H, D;
    int P;                   // workgroups per team (hidden-unit slices)
    int BG;                  // batch rows per team
    int NGB;                 // batch groups
    int kch;                 // K chunks of H
    int kchp;                // chunks resident in LDS (kch padded to whole batches per wave)
    int nbatch;              // chunk batches per wave
    int part_bufs;           // 1 or 2 partial-sum buffers in LDS
    int poll_sleep;          // s_sleep units (64 clocks each) between re-reads of stale words
    int pace;                // wall-clock ticks from the end of a step to the first read of the next
    int s_begin, s_end;      // steps handled by this launch
    int map_xcd;             // 1: place a team's workgroups on the same XCDs
    int vec;                 // 16-byte vector loads are aligned
    int wreg;                // W_hh fragments in registers (RecGeom::wreg; selects the kernel)
    // fused input projection (ncx > 0): G is not read; x_t W_ih^T + b_ih + b_hh
    // is computed in the step from these
    int ncx;                 // input chunks per wave (0: use G)
    int I;                   // input width of this layer
    const void *x;           // [T, B, I] dtype
    const void *wih[2];      // [4H, I] per direction, dtype
    const void *b_ih[2];     // [4H] dtype or NULL
    const void *b_hh[2];
    long long timeout_ticks; // wait timeout in wall_clock64 ticks
    int mode;                // recurrent mode of k_rec_step: 0 LSTM, 1 GRU, 2 RNN_TANH, 3 RNN_RELU
};

constexpr int kMaxTeams = 64;

// The layer wavefront (rec_wave.hip): every layer of a unidirectional stack in
// one persistent launch, two workgroups per CU, layer l > 0 multiplying layer
// l-1's h_t (read from its exchange words) as its input; layer 0 multiplies
// x_t.  Teams of at most 16 batch rows, U = 4 NT units per workgroup.
constexpr int kMaxPipeLayers = 4;
struct WaveArgs {
    const void *x;                          // [T, B, I] dtype: layer 0's input
    const void *wih[kMaxPipeLayers];        // [4H, in_l] dtype (in_0 = I, else H)
    const void *whh[kMaxPipeLayers];        // [4H, H] dtype
    const void *b_ih[kMaxPipeLayers];       // [4H] dtype or NULL (no bias)
    const void *b_hh[kMaxPipeLayers];
    const void *h0;                         // [L, B, H] dtype, or NULL (zeros)
    const float *c0;                        // [L, B, H] or NULL
    void *Y;                                // [T, B, H] dtype: output of the last layer
    void *hn;                               // [L, B, H] dtype or NULL
    float *cn;                              // [L, B, H] or NULL
    uint32_t *xbuf[kMaxPipeLayers];         // per layer: [slots][NGB][kch * 256] exchange words, zeroed;
                                            // T slots, or 2 for the last layer
    unsigned *status;
    int L, T, B, H, I;
    int P, BG, NGB, kch;
    int ncx0;                               // layer 0's input chunks per wave
    int map_xcd;                            // 1: a team's workgroups on 8 / NGB XCDs
    int poll_sleep, pace, vec;
    long long timeout_ticks;
};
// Small-batch recurrence (rec_xcd.hip): one layer, B <= 16 rows, direction d's
// 32-unit workgroups on XCD d (a launch of 8 P workgroups of 512 threads, id
// % 8 = XCD); hoisted projection G; W_hh in registers.  Shapes: K <= 8 waves
// x 4 chunks (H <= 1024 bf16 / 512 fp32), at most 32 workgroups per direction.
bool xcd_shape_ok(int H, int B, int D, int dtype);
int xcd_workgroups(int H);
hipError_t xcd_max_coresident(int dtype, int *blocks_per_cu);
hipError_t launch_xcd(const RecArgs &a, int dtype, hipStream_t s);

// Large-batch recurrence with W_hh held once across the chip and h exchanged
// through a two-slot ring of tagged words (rec_res.hip).  res_shape_ok:
// bf16, H one of 256, 512, 1024, 1536, 2048, (ceil(B/128) * D) groups x H/16
// unit slices <= cus workgroups; it returns the groups, the slices and
// whether the XCD-aware order applies.  The launch takes NGB = groups,
// P = slices, map_xcd as returned, and xbuf pointing at res_ring_bytes(H,
// groups) zeroed bytes.
bool res_shape_ok(int H, int B, int D, int dtype, int cus, int *groups, int *slices, int *map_xcd);
size_t res_ring_bytes(int H, int groups);
hipError_t res_max_coresident(int H, int *blocks_per_cu);
hipError_t launch_res(const RecArgs &a, hipStream_t s);

// The wavefront applies when W_hh's K fits 4 waves x 8 chunks, layer 0's
// input width fits 8 chunks per wave (ncx0: its chunks per wave), and H and
// the input width are multiples of 16 bytes.
bool wave_shape_ok(int H, int I, int dtype, int *ncx0);
// nt: 4 nt units per workgroup (1, 2 or 4); lpw: layers per workgroup (1, or
// 2 for a two-layer stack: both layers' unit slice in one 512-thread workgroup)
hipError_t wave_max_coresident(int nt, int dtype, int lpw, int *blocks_per_cu);
hipError_t launch_wave(const WaveArgs &a, int nt, int dtype, int lpw, hipStream_t s);

// Recurrent tile: 4 waves split (4/WK) ways over batch tiles and WK ways over
// K; each wave owns MTW 16-row batch tiles; NT 16-column tiles of gate rows
// (4 hidden units each, gates interleaved) make U = 4*NT units per workgroup.
struct RecTile {
    int WK, MTW, NT;
};

constexpr size_t kRecLdsLimit = 160 * 1024 - 64;  // leaves room for static LDS

// LDS geometry of a recurrent tile for hidden size H.
struct RecGeom {
    int kch, kchp, nbatch, part_bufs;
    int wreg;  // 1: each wave holds its W_hh fragments in registers; LDS holds partial sums only
    size_t smem;
};
RecGeom rec_geom(RecTile t, int H, int dtype, bool want_two_partial_buffers);
int rec_rows_per_wg(RecTile t);
bool rec_tile_supported(RecTile t);

// variant: 0 automatic, 1 128x128 tiles, 2 256x256 tiles, 3 256x256 tiles with direct-to-LDS loads
hipError_t launch_proj(const ProjArgs &a, int dtype, int variant, hipStream_t s);
// K-split depth for an fp32 M x N x K product with few output tiles: a chunk
// (multiple of 64) that gives about one 256x256 tile per CU, or 0 (no split).
int proj_kchunk(int M, int N, int K);
// out[i] = sum over s < ns of part[s * slab + i], in the order s = 0, 1, ...; out is dtype
hipError_t launch_ksum(const float *part, int ns, size_t slab, size_t n, void *out, int dtype, hipStream_t s);
// Name of the projection kernel launch_proj picks for an M x N x K product
// over D directions, given 16-byte aligned operands.
const char *proj_kernel_name(int M, int N, int K, int D, int dtype, int variant);
hipError_t launch_rec(const RecArgs &a, RecTile t, size_t smem, int dtype, bool cooperative, hipStream_t s);
hipError_t rec_max_coresident(RecTile t, size_t smem, int dtype, bool wreg, bool fused, bool wide,
                              int *blocks_per_cu);
// input chunks per wave of the tile's fused-projection variant (0: none)
int rec_fused_chunks(RecTile t);
// The k_rec instance for tile t (rec_f32.hip, rec_bf16.hip, rec_bf16_wide.hip):
// W_hh in registers or LDS, fused or hoisted projection; nullptr if none.
const void *rec_kernel_f32(RecTile t, bool wreg, bool fused);
const void *rec_kernel_bf16(RecTile t, bool wreg, bool fused);
const void *rec_kernel_bf16_wide(RecTile t, bool wreg, bool fused);
// ----------------------------------------------------------------- backward
// One backward step (sb = 0 is the last step of each direction's scan) of one
// layer, all directions.
struct BwdCellArgs {
    const float *acts;  // [T, B, D, 5, H] saved by the training forward (i, f, g, o, c)
    const float *c0;    // [D, B, H] of this layer, or NULL (zeros)
    const float *dY;    // [T, B, D*H] gradient of this layer's output
    const float *dhn;   // [D, B, H] gradient of h_n of this layer, or NULL
    const float *dcn;   // [D, B, H] gradient of c_n of this layer, or NULL
    void *dz;           // [T, B, D, 4H] gradient of the pre-activations (gradient dtype), written at each step's time
    float *dc;          // [D, B, H] cell-state gradient carried backwards (read and written)
    const int *len;     // [B] valid steps per row, or NULL (all T)
    float *dhc;         // [D, B, H] with len: the gradient of h carried through padded steps
    int T, B, H, D;
};
// the recurrent product of step sb: dz_t W_hh
struct BwdMmArgs {
    const void *dz;     // [T, B, D, 4H], gradient dtype
    const void *whT;    // [D, H, 4H] transposed W_hh, gradient dtype
    int T, B, H, D, sb;
    // ksplit 2: each 16x16 tile's K = 4H is split between two workgroups; the
    // second hands its partial sums to the first through pbuf ([D][tiles]
    // [256] words of (tag << 32 | fp32 bits), zeroed before the first launch
    // of a call), tagged with this launch's tag (unique within the call, not
    // 0); a wait that outlasts timeout_ticks sets bit 1 of *status
    int ksplit;
    unsigned tag;
    unsigned long long *pbuf;
    unsigned *status;
    long long timeout_ticks;
};
// The backward pass stores dz and multiplies it in the gradient dtype gdt:
// bf16 (fp32 accumulation; the cell math stays fp32) for bf16 parameters
// with an even H (whole 16-byte fragments over K = 4H), fp32 otherwise.
// The first backward step of a layer (dh = dY + dh_n), elementwise.
hipError_t launch_bwd_cell(const BwdCellArgs &a, int gdt, hipStream_t s);
// Backward step a.sb: the recurrent product, then the cell update of step
// a.sb + 1, or dh0 ([D, B, H], dtype; NULL = not wanted) after the last step.
// With a.ksplit = 2 every workgroup of the launch must be resident at once
// (two per tile; the caller keeps the grid within one per CU).
hipError_t launch_bwd_step(const BwdMmArgs &a, const BwdCellArgs &c, void *dh0, int gdt, int dtype, hipStream_t s);
// out[c * ld_out + r] = in[r * ld_in + c] (rows x cols, in_dtype -> out_dtype);
// with bT > 0 (rows = bT * bB) the input rows are batch-first: row r = t*bB + b
// of the result reads input row b*bT + t
hipError_t launch_transpose(const void *in, size_t ld_in, int rows, int cols, void *out, size_t ld_out, int in_dtype,
                            int out_dtype, hipStream_t s, int bT = 0, int bB = 0);
// rows of width elements between [B][T] and [T][B] order (to_time_major:
// batch-first in, time-major out), converting in_dtype -> out_dtype
hipError_t launch_permute_rows(const void *in, void *out, int T, int B, int width, int in_dtype, int out_dtype,
                               bool to_time_major, hipStream_t s);
// [H][T*B] in out_dtype: h_prev of direction d for every (t, b), from the
// layer output Y or h0d ([B][H] or NULL), both dtype (bf16 -> fp32 allowed);
// with per-row lengths (len, or NULL) a padded predecessor's h is h0d's
hipError_t launch_hprev_t(const void *Y, size_t ldy, const void *h0d, const int *len, int T, int B, int H, int d,
                          void *out, int dtype, int out_dtype, hipStream_t s, bool batch_first = false);
// part[c][col] (c < the chunk count launched, at most nchunks) = sum over
// the rows of chunk c of a[r * ld + col]; rows split into ceil(rows /
// nchunks)-row chunks, each summed in row order
hipError_t launch_colsum_part(const void *a, size_t ld, int rows, int cols, int nchunks, float *part, int dtype,
                              hipStream_t s);
hipError_t launch_cast_to(const float *in, void *out, size_t n, int dtype, hipStream_t s);
hipError_t launch_cast_from(const void *in, float *out, size_t n, int dtype, hipStream_t s);
// Training dropout of one layer's output y ([T][B][width] of dtype, or
// [B][T][width] when batch_first): xd = the next layer's input in y's layout,
// keep = one byte per element in time-major order (the order of the draw's
// element index); thr = ceil(p * 2^53), scale = 1 / (1 - p) (0 when p = 1).
hipError_t launch_dropout_fwd(const void *y, void *xd, unsigned char *keep, int T, int B, int width,
                              unsigned long long seed, unsigned long long call, int layer, unsigned long long thr,
                              float scale, int dtype, bool batch_first, hipStream_t s);
// g[e] = keep[e] ? g[e] * scale : 0
hipError_t launch_dropout_bwd(float *g, const unsigned char *keep, size_t n, float scale, hipStream_t s);

// Zero the y row of (t, b) for every t >= len[b] (padded steps of variable-length rows).
hipError_t launch_mask_padded(void *y, const int *len, int T, int B, size_t row_bytes, bool batch_first, hipStream_t s);
hipError_t launch_fill_u32(unsigned *p, size_t n, unsigned v, hipStream_t s);
// Row-padded parameter copies: dst (rows x cols, dtype) = the first `valid`
// rows of src (row-major, cols wide), zeros below.  Any number of jobs.
struct PadJob {
    const void *src;
    void *dst;
    int valid, rows, cols;
};
hipError_t launch_pad_rows(const PadJob *jobs, int n, int dtype, hipStream_t s);
// One recurrent step (a.s_begin) as a GEMM with the cell update fused
// (k_rec_step); reads h_{t-1} from a.Y / a.h0 and carries c in a.cstate.
// rec_step_gemm_ok: its alignment and 31-bit offset requirements hold.
bool rec_step_gemm_ok(const RecArgs &a, int dtype);
// Batch rows per workgroup of k_rec_step (64 with two K slices, or 128).
int rec_step_rows(int B);
hipError_t launch_rec_step_gemm(const RecArgs &a, int dtype, hipStream_t s);

// The forward pass behind lstm_forward (every recurrent mode); own_ws: the
// workspace is the library's own device array (lstm_forward_static) rather
// than caller memory, so it is not checked as caller memory.
lstm_status forward_dispatch(lstm_plan *p, const void *x, const void *h0, const float *c0,
                             const void *const *weights, int T, int B, int layers, int bidir, void *y, void *h_n,
                             float *c_n, void *workspace, size_t workspace_bytes, void *stream, bool own_ws);

}  // namespace lstm_amd
