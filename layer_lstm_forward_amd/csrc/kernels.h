// kernels.h -- host-side interface of the gfx950 kernels (internal; the public
// ABI is include/lstm.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace lstm_amd {

enum DType { DT_F32 = 0, DT_BF16 = 1 };

// G[m][d*N + n] = sum_k X[m][k] * W_d[n][k] + b_ih_d[n] + b_hh_d[n]
//   X   [M, K] with row stride ldx (elements), dtype
//   W_d [N, K] row-major, dtype; N = 4H; d = 0..D-1 (blockIdx.z)
//   G   [M, D*N] float32
struct ProjArgs {
    const void *X;
    const void *W[2];
    const void *b_ih[2];
    const void *b_hh[2];
    float *G;
    int M, N, K, ldx, D;
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
    unsigned long long *xbuf;  // h exchange: [2][D][NGB] regions of (ROWS/16)*kch*256 tagged words
    unsigned tag_base;       // tags of this layer are tag_base + s + 1
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
    long long timeout_ticks; // wait timeout in wall_clock64 ticks
};

constexpr int kMaxTeams = 64;

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
    size_t smem;
};
RecGeom rec_geom(RecTile t, int H, int dtype, bool want_two_partial_buffers);
int rec_rows_per_wg(RecTile t);
bool rec_tile_supported(RecTile t);

// variant: 0 automatic, 1 128x128 tiles, 2 256x256 tiles, 3 256x256 tiles with direct-to-LDS loads
hipError_t launch_proj(const ProjArgs &a, int dtype, int variant, hipStream_t s);
// Name of the projection kernel launch_proj picks for an M x N x K product
// over D directions, given 16-byte aligned operands.
const char *proj_kernel_name(int M, int N, int K, int D, int dtype, int variant);
hipError_t launch_rec(const RecArgs &a, RecTile t, size_t smem, int dtype, bool cooperative, hipStream_t s);
hipError_t rec_max_coresident(RecTile t, size_t smem, int dtype, int *blocks_per_cu);
hipError_t launch_fill_u32(unsigned *p, size_t n, unsigned v, hipStream_t s);
// One recurrent step (a.s_begin) as a GEMM with the cell update fused
// (k_rec_step); reads h_{t-1} from a.Y / a.h0 and carries c in a.cstate.
// rec_step_gemm_ok: its alignment and 31-bit offset requirements hold.
bool rec_step_gemm_ok(const RecArgs &a, int dtype);
hipError_t launch_rec_step_gemm(const RecArgs &a, int dtype, hipStream_t s);

}  // namespace lstm_amd
