// rec.h -- the persistent recurrence kernel k_rec, a template over the
// element type, the tile and the exchange word format.  Its instances are
// compiled in three translation units (rec_f32.hip, rec_bf16.hip,
// rec_bf16_wide.hip), each exporting a table from tile to kernel.
#pragma once

#include "device.h"
#include "kernels.h"

namespace lstm_amd {

// Recurrent tiles (WK, MTW, NT) with a kernel instance, and the subset with a
// fused-projection instance and its input chunks per wave.
#define LSTM_REC_TILES(X) \
    X(4, 1, 1) X(4, 1, 2) X(4, 1, 4) X(2, 1, 1) X(2, 1, 2) X(2, 1, 4) X(1, 1, 1) X(1, 1, 2) X(1, 1, 4) \
    X(1, 4, 1) X(1, 4, 2)
#define LSTM_REC_FUSED_TILES(X) X(4, 1, 1) X(4, 1, 2) X(4, 1, 4) X(2, 1, 1) X(2, 1, 2) X(2, 1, 4)
#define LSTM_FX_OF(nt) ((nt) == 4 ? 4 : 8)

// ===========================================================================
// Recurrence.  A team of P workgroups shares one direction and one group of
// BG batch rows; workgroup p owns hidden units [p*U, p*U+U) and therefore the
// 4U rows {q*H + j : q in i,f,g,o} of W_hh, kept in LDS as MFMA fragments
// (gate rows interleaved: local column n = 4*u + q).  Per step:
//   1. prefetch the projection G[t] for the cells this thread updates;
//   2. S = h_{t-1} W_slice^T: the four waves split over batch tiles and K;
//      each wave fetches its h_{t-1} fragments from the exchange buffer of
//      compact tagged words (re-reading words until they carry step t-1's
//      tag bit; at t = 0 plain loads of h0) and feeds them to the matrix
//      cores;
//   3. partial sums meet in LDS; each thread reduces the gate pre-activations
//      of a pair of adjacent units of one batch row, applies sigma/tanh,
//      updates c (kept in registers across steps) and writes h_t to y, to the
//      exchange buffer with the next tag, and at the end to h_n and c_n.
// One launch can run every step of the layer (persistent: all workgroups must
// be co-resident, which the cooperative launch guarantees) or just one.
// With RW, each wave keeps the W_hh fragments of its own K range in
// registers for the whole launch (used when that range is one batch of CB
// chunks): the matrix cores then never wait on LDS, and LDS holds only the
// partial sums.
// With FX > 0 the input projection is fused instead of hoisted: each wave
// also keeps the W_ih fragments of its share of the input width in registers
// (at most FX chunks) and multiplies x_t by them right after issuing the
// reads of h_{t-1}, i.e. while the matrix cores would otherwise wait for the
// exchange; both biases are added in the epilogue and G is not used.  The
// same equation block splits the gate pre-activation into the x_t and h_{t-1}
// products; here they share one accumulator.
// XW selects the wide bf16 exchange words (one value per word; device.h), for
// recurrences whose published h is not bounded by 1; fp32 ignores it.
// ===========================================================================
template <class DT, int WK, int MTW, int NT, int CB, bool RW, int FX, bool XW>
__global__ __launch_bounds__(256) void k_rec(RecArgs a) {
    using S = typename DT::S;
    constexpr bool FUSED = FX > 0;
    static_assert(!FUSED || RW, "the fused projection keeps W_hh in registers");
    constexpr bool BF = sizeof(S) == 2;
    constexpr int XF = !BF ? XF_F32 : XW ? XF_WIDE : XF_PAIR;  // exchange word format
    constexpr bool WIDE = XF == XF_WIDE;
    constexpr int NWL = WIDE ? 2 : 1;  // 16-byte exchange loads per fragment
    constexpr int WM = 4 / WK;
    constexpr int MT = WM * MTW;
    constexpr int ROWS = 16 * MT;
    constexpr int NCOL = 16 * NT;
    constexpr int U = 4 * NT;
    constexpr int PSTR = NCOL + 4;
    constexpr int CELLS = ROWS * U;
    constexpr int CPT = (CELLS + 255) / 256;
    constexpr int EW = XF == XF_PAIR ? 2 : 1;  // K values per exchange word
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_bad;
    u32x4 *Wf = reinterpret_cast<u32x4 *>(smem);
    float *part0 = reinterpret_cast<float *>(smem + (RW ? (size_t)0 : (size_t)a.kchp * NT * 1024));
    const size_t part_stride = (size_t)WK * ROWS * PSTR;  // floats per partial buffer

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w / WK, wk = w % WK;
    const int nteams = a.NGB * a.D;
    int team, p;
    {
        const int bid = blockIdx.x;
        if (a.map_xcd) {
            const int X = 8 / nteams;  // XCDs per team (dispatch is round-robin over 8 XCDs)
            team = (bid & 7) / X;
            p = (bid >> 3) * X + (bid & 7) % X;
        } else {
            team = bid / a.P;
            p = bid % a.P;
        }
    }
    const int H = a.H, B = a.B, T = a.T, D = a.D, kch = a.kch;
    const int d = team % D, gb = team / D;
    const int b0 = gb * a.BG, rows = min(a.BG, B - b0);
    const int j0 = p * U, units = min(U, H - j0);
    const size_t ldy = (size_t)D * H;
    const size_t ldg = (size_t)D * 4 * H;
    const bool vec = a.vec != 0;

    // Resident W_hh slice as fragments: [chunk][n-tile][lane] x 16 bytes,
    // zero beyond H and for the padding chunks up to kchp; in registers
    // (this wave's chunks [wk*CB, wk*CB + CB)) or in LDS.
    u32x4 wreg[RW ? CB : 1][NT];
    if constexpr (RW) {
        const S *W = static_cast<const S *>(a.whh[d]);
#pragma unroll
        for (int ci = 0; ci < CB; ++ci)
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int n = j * 16 + (lane & 15), u = n >> 2, q = n & 3;
                const int k = (wk * CB + ci) * DT::KC + (lane >> 4) * DT::PER16;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (u < units && k < H) v = load_frag<DT>(W + (size_t)(q * H + j0 + u) * H, k, H, vec);
                wreg[ci][j] = v;
            }
    } else {
        const S *W = static_cast<const S *>(a.whh[d]);
        const int nfrag = a.kchp * NT * 64;
        for (int f = tid; f < nfrag; f += 256) {
            const int ln = f & 63, nt = (f >> 6) % NT, c = (f >> 6) / NT;
            const int n = nt * 16 + (ln & 15), u = n >> 2, q = n & 3;
            const int k = c * DT::KC + (ln >> 4) * DT::PER16;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (u < units && k < H) v = load_frag<DT>(W + (size_t)(q * H + j0 + u) * H, k, H, vec);
            Wf[f] = v;
        }
    }

    // Fused projection: W_ih fragments of input chunks [wk*ncx, wk*ncx + ncx)
    // (ncx <= FX; the chunks past the input width are zero).
    const int ncx = FUSED ? a.ncx : 0;
    u32x4 wx[FUSED ? FX : 1][NT];
    if constexpr (FUSED) {
        const S *Wi = static_cast<const S *>(a.wih[d]);
#pragma unroll
        for (int cx = 0; cx < FX; ++cx)
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int n = j * 16 + (lane & 15), u = n >> 2, q = n & 3;
                const int k = (wk * ncx + cx) * DT::KC + (lane >> 4) * DT::PER16;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (cx < ncx && u < units && k < a.I) v = load_frag<DT>(Wi + (size_t)(q * H + j0 + u) * a.I, k, a.I, true);
                wx[cx][j] = v;
            }
    }

    // Cells of this thread: (batch row cm, hidden unit cu); adjacent lanes hold
    // adjacent units of one row.
    // With per-row lengths a cell is active at time t only if t < its row's
    // length; otherwise c and h stay as they are (hreg keeps h), y gets 0.
    // The GRU (a.mode 1) also needs its cell's h_{t-1} in hreg, and b_hn.
    int cm[CPT], cu[CPT], clen[CPT];
    bool cv[CPT];
    float creg[CPT], hreg[CPT], bhn[CPT];
    const bool keep_h = a.len || a.mode == 1;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int e = tid + 256 * i;
        cm[i] = e / U;
        cu[i] = e % U;
        cv[i] = e < CELLS && cm[i] < rows && cu[i] < units;
        creg[i] = 0.f;
        hreg[i] = 0.f;
        bhn[i] = 0.f;
        clen[i] = T;
        if (cv[i]) {
            const size_t si = ((size_t)d * B + b0 + cm[i]) * H + j0 + cu[i];
            if (a.s_begin == 0) {
                creg[i] = a.c0 ? a.c0[si] : 0.f;
                if (keep_h && a.h0) hreg[i] = DT::to_f(static_cast<const S *>(a.h0)[si]);
            } else {
                creg[i] = a.cstate[si];
                if (keep_h) hreg[i] = a.hstate[si];
            }
            if (a.len) clen[i] = a.len[b0 + cm[i]];
            if (a.mode == 1 && a.b_hh[d]) bhn[i] = DT::to_f(static_cast<const S *>(a.b_hh[d])[(size_t)2 * H + j0 + cu[i]]);
        }
    }
    if (tid == 0) s_bad = 0;
    // fused projection: b_ih + b_hh of this thread's cells
    float bias[FUSED ? CPT : 1][4];
    if constexpr (FUSED) {
        const S *bi = static_cast<const S *>(a.b_ih[d]), *bh = static_cast<const S *>(a.b_hh[d]);
#pragma unroll
        for (int i = 0; i < CPT; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = q * H + j0 + (cv[i] ? cu[i] : 0);
                bias[i][q] = bi ? DT::to_f(bi[r]) + DT::to_f(bh[r]) : 0.f;
            }
    }

    // G[t] of this thread's cells, loaded two steps ahead: older loads hold
    // up the in-order wait on the exchange loads, so they are issued early.
    // Steps alternate between two register sets (the loop below is unrolled
    // by two) so that no register with a load in flight is ever copied, and
    // every load is unconditional (a dead cell or a step past the end reads
    // a valid clamped address and the value is never used): a copy or a
    // conditional join would make the compiler wait for the loads at once.
    float gA[FUSED ? 1 : CPT][4], gB[FUSED ? 1 : CPT][4];
    auto load_g = [&](int step, float (&g)[FUSED ? 1 : CPT][4]) {
        const int tg = d == 0 ? step : T - 1 - step;
        const bool in = step < a.s_end;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const bool ok = in && cv[i];
            const float *gp = a.G + trow(ok ? tg : 0, b0 + (ok ? cm[i] : 0), T, B, a.bfirst) * ldg +
                              (size_t)d * 4 * H + j0 + (ok ? cu[i] : 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) g[i][q] = gp[(size_t)q * H];
        }
    };
    // Fused projection: x_t fragments of this wave's rows and input chunks,
    // loaded two steps ahead in the same way (one buffer resource per time
    // slice; rows past the batch group and chunks past the input read zeros).
    const int mw0 = wm * MTW * 16 + (lane & 15);
    u32x4 xA[FUSED ? FX : 1][MTW], xB[FUSED ? FX : 1][MTW];
    auto load_x = [&](int step, u32x4 (&xf)[FUSED ? FX : 1][MTW]) {
        const int st = step < a.s_end ? step : a.s_begin;
        // wave-uniform by construction; said explicitly so that the resource
        // stays in scalar registers (else every load becomes a waterfall loop)
        const int tx = __builtin_amdgcn_readfirstlane(d == 0 ? st : T - 1 - st);
        // rows of batch rows b0.. at time tx: consecutive (time-major) or T
        // rows apart (batch_first)
        const size_t xstride = a.bfirst ? (size_t)T * a.I : (size_t)a.I;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<S *>(static_cast<const S *>(a.x) + trow(tx, 0, T, B, a.bfirst) * a.I), (short)0,
            (int)(((size_t)(B - 1) * xstride + a.I) * sizeof(S)), 0x00020000);
#pragma unroll
        for (int cx = 0; cx < FX; ++cx)
#pragma unroll
            for (int i = 0; i < MTW; ++i) {
                const int m = mw0 + 16 * i;
                const int k = (wk * ncx + cx) * DT::KC + (lane >> 4) * DT::PER16;
                const bool ok = cx < ncx && m < rows && k < a.I;
                xf[cx][i] = __builtin_amdgcn_raw_buffer_load_b128(
                    r, ok ? (int)((((size_t)(b0 + m)) * xstride + k) * sizeof(S)) : 0x7FFFFFF0, 0, 0);
            }
    };
    if constexpr (FUSED) {
        load_x(a.s_begin, xA);
        load_x(a.s_begin + 1, xB);
    } else {
        load_g(a.s_begin, gA);
        load_g(a.s_begin + 1, gB);
    }
    __syncthreads();

    const int nb = RW ? 1 : a.nbatch;              // chunk batches per wave
    const int cw0 = wk * nb * CB;                  // first chunk of this wave
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const int mw = wm * MTW * 16 + (lane & 15);    // this lane's team row in tile i: mw + 16 i
    const int ksub = (lane >> 4) * DT::PER16;      // this lane's K offset inside a chunk
    const size_t region = (size_t)MT * kch * 256 * NWL;  // 32-bit exchange words per team
    uint32_t *const xb32 = reinterpret_cast<uint32_t *>(a.xbuf);
    // Optional read pacing: every wave waits `pace` wall-clock ticks after the
    // barrier that ends its workgroup's step s-1 before its first read of the
    // others' h_{s-1}, so that reads do not reach memory ahead of the data.
    long long t_pub = 0;

    // one step; false when a wait gave up (the kernel then leaves)
    auto step = [&](const int s, float (&gcur)[FUSED ? 1 : CPT][4], u32x4 (&xcur)[FUSED ? FX : 1][MTW])
        __attribute__((always_inline)) -> bool {
        const int t = d == 0 ? s : T - 1 - s;
        float *part = part0 + (a.part_bufs == 2 ? (size_t)(s & 1) * part_stride : 0);

        f32x4 acc[MTW][NT];
#pragma unroll
        for (int i = 0; i < MTW; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        bool wave_ok = true;
        // x_t W_ih^T for this wave's input chunks (fused projection)
        auto mma_x = [&]() {
            if constexpr (FUSED) {
#pragma unroll
                for (int cx = 0; cx < FX; ++cx)
                    if (cx < ncx)
#pragma unroll
                        for (int i = 0; i < MTW; ++i)
#pragma unroll
                            for (int j = 0; j < NT; ++j) acc[i][j] = mma_chunk(DT{}, acc[i][j], xcur[cx][i], wx[cx][j]);
            }
        };

        if (s == 0) {
            mma_x();
            if (a.h0) {
                const S *hs = static_cast<const S *>(a.h0) + (size_t)d * B * H;
                for (int bi = 0; bi < nb; ++bi)
#pragma unroll
                    for (int ci = 0; ci < CB; ++ci) {
                        const int c = cw0 + bi * CB + ci;
                        u32x4 af[MTW];
                        const int k = c * DT::KC + ksub;
#pragma unroll
                        for (int i = 0; i < MTW; ++i) {
                            const int m = mw + 16 * i;
                            af[i] = (m < rows && k < H) ? load_frag<DT>(hs + (size_t)(b0 + m) * H, k, H, vec) : zero;
                        }
#pragma unroll
                        for (int j = 0; j < NT; ++j) {
                            const u32x4 bw = RW ? wreg[RW ? ci : 0][j] : Wf[(c * NT + j) * 64 + lane];
#pragma unroll
                            for (int i = 0; i < MTW; ++i) acc[i][j] = mma_chunk(DT{}, acc[i][j], af[i], bw);
                        }
                    }
            }
        } else {
            const unsigned tb = xc_tag(a.xpar, s - 1);  // written at step s-1
            const __amdgpu_buffer_rsrc_t xr =
                xcrsrc(xb32 + ((size_t)(((s - 1) & 1) * D + d) * a.NGB + gb) * region, (unsigned)(region * 4));
            if (s > a.s_begin && a.pace > 0)
                while (wall_clock64() - t_pub < a.pace) __builtin_amdgcn_s_sleep(1);
            for (int bi = 0; bi < nb && wave_ok; ++bi) {
                const int c0 = cw0 + bi * CB;
                // Each lane reads its fragment (four words, or eight wide
                // words) with NWL 16-byte loads; for each of them the 64
                // lanes of a wave read 1 KB in a row.
                u32x4 wd[CB][MTW][NWL];
                unsigned off[CB][MTW];
                bool lv[CB][MTW][4 * NWL];
#pragma unroll
                for (int ci = 0; ci < CB; ++ci)
#pragma unroll
                    for (int i = 0; i < MTW; ++i) {
                        const int c = c0 + ci, m = mw + 16 * i;
#pragma unroll
                        for (int e = 0; e < 4 * NWL; ++e) lv[ci][i][e] = m < rows && c * DT::KC + ksub + e * EW < H;
                        off[ci][i] = lv[ci][i][0] ? (unsigned)((((wm * MTW + i) * kch + c) * 64 + lane) * 16 * NWL)
                                                  : 0x7FFFFFF0u;  // out of range: reads zeros, no memory access
                    }
#pragma unroll
                for (int ci = 0; ci < CB; ++ci)
#pragma unroll
                    for (int i = 0; i < MTW; ++i)
#pragma unroll
                        for (int h = 0; h < NWL; ++h) wd[ci][i][h] = xload2(xr, off[ci][i] + 16u * h);
                if (bi == 0) mma_x();  // overlaps the reads of h_{t-1}
                // a dead word (padding row or K past H) counts as ready; its
                // value (zero, or the fp32 tag bit alone) meets zero W rows or
                // a discarded output row
                const unsigned tpat = tb << xc_shift(XF);
                auto settle = [&](int ci, int i) {
#pragma unroll
                    for (int h = 0; h < NWL; ++h) {
                        if (!lv[ci][i][4 * h + 0]) wd[ci][i][h].x = tpat;
                        if (!lv[ci][i][4 * h + 1]) wd[ci][i][h].y = tpat;
                        if (!lv[ci][i][4 * h + 2]) wd[ci][i][h].z = tpat;
                        if (!lv[ci][i][4 * h + 3]) wd[ci][i][h].w = tpat;
                    }
                };
                bool mine = true;
#pragma unroll
                for (int ci = 0; ci < CB; ++ci)
#pragma unroll
                    for (int i = 0; i < MTW; ++i) {
                        settle(ci, i);
#pragma unroll
                        for (int h = 0; h < NWL; ++h) mine = mine & xc_ok<XF>(wd[ci][i][h], tb);
                    }
                if (!__all(mine)) {
                    // slow path: back off, then re-read only the fragments that are stale
                    unsigned spins = 0;
                    const long long t0 = wall_clock64();
                    do {
                        if ((++spins & 31u) == 0) {
                            const unsigned st = __builtin_amdgcn_readfirstlane(
                                __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                            if (st != 0u) {
                                wave_ok = false;
                                break;
                            }
                            if (wall_clock64() - t0 > a.timeout_ticks) {
                                if (lane == 0)
                                    __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
                                wave_ok = false;
                                break;
                            }
                        }
                        for (int z = 0; z < a.poll_sleep; ++z) __builtin_amdgcn_s_sleep(1);
                        // re-read the stale fragments; every load is issued
                        // (a current fragment's goes out of range: zeros, no
                        // memory access) before any is waited for, so one
                        // retry costs one round trip however many are stale
                        bool stale[CB][MTW][NWL];
                        u32x4 re[CB][MTW][NWL];
#pragma unroll
                        for (int ci = 0; ci < CB; ++ci)
#pragma unroll
                            for (int i = 0; i < MTW; ++i)
#pragma unroll
                                for (int h = 0; h < NWL; ++h) {
                                    stale[ci][i][h] = !xc_ok<XF>(wd[ci][i][h], tb);
                                    re[ci][i][h] = xload2(xr, stale[ci][i][h] ? off[ci][i] + 16u * h : 0x7FFFFFF0u);
                                }
                        mine = true;
#pragma unroll
                        for (int ci = 0; ci < CB; ++ci)
#pragma unroll
                            for (int i = 0; i < MTW; ++i) {
#pragma unroll
                                for (int h = 0; h < NWL; ++h)
                                    if (stale[ci][i][h]) wd[ci][i][h] = re[ci][i][h];
                                settle(ci, i);
#pragma unroll
                                for (int h = 0; h < NWL; ++h) mine = mine & xc_ok<XF>(wd[ci][i][h], tb);
                            }
                    } while (!__all(mine));
                    if (!wave_ok) break;
                }
#pragma unroll
                for (int ci = 0; ci < CB; ++ci) {
                    u32x4 bw[NT];
#pragma unroll
                    for (int j = 0; j < NT; ++j) bw[j] = RW ? wreg[RW ? ci : 0][j] : Wf[((c0 + ci) * NT + j) * 64 + lane];
#pragma unroll
                    for (int i = 0; i < MTW; ++i) {
                        // the fragment's values without their tag bits
                        u32x4 af = wd[ci][i][0];
                        if constexpr (WIDE) {
                            const u32x4 hi = wd[ci][i][NWL - 1];
                            af = u32x4{xc_wide_pair(af.x, af.y), xc_wide_pair(af.z, af.w), xc_wide_pair(hi.x, hi.y),
                                       xc_wide_pair(hi.z, hi.w)};
                        } else if constexpr (XF == XF_PAIR) {
                            af = u32x4{xc_pair_value(af.x), xc_pair_value(af.y), xc_pair_value(af.z),
                                       xc_pair_value(af.w)};
                        }
#pragma unroll
                        for (int j = 0; j < NT; ++j) acc[i][j] = mma_chunk(DT{}, acc[i][j], af, bw[j]);
                    }
                }
            }
        }

#pragma unroll
        for (int i = 0; i < MTW; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = (wm * MTW + i) * 16 + 4 * (lane >> 4) + v;
                    const int n = j * 16 + (lane & 15);
                    part[(wk * ROWS + m) * PSTR + n] = acc[i][j][v];
                }
        if (!wave_ok) s_bad = 1;
        __syncthreads();
        if (s_bad) return false;  // a wait gave up: leave (every workgroup drains the same way)

        const unsigned tb_out = xc_tag(a.xpar, s);
        uint32_t *xo = xb32 + ((size_t)((s & 1) * D + d) * a.NGB + gb) * region;
        const bool publish = s + 1 < T;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            // every lane of the wave takes part in the shuffle below
            float hv = 0.f;
            S hs = (S)0;
            if (cv[i]) {
                const float *pp = &part[cm[i] * PSTR + 4 * cu[i]];
                const f32x4 sum = lds_sum_f32x4<WK>(pp, ROWS * PSTR);
                float pre[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if constexpr (FUSED) pre[q] = bias[i][q];
                    else pre[q] = gcur[i][q];
                }
                float ig = 0.f, fg = 0.f, gg = 0.f, og = 0.f, cn = creg[i];
                if (a.mode == 0) {
                    ig = sigmoid_f(sum.x + pre[0]);
                    fg = sigmoid_f(sum.y + pre[1]);
                    gg = tanh_f(sum.z + pre[2]);
                    og = sigmoid_f(sum.w + pre[3]);
                    cn = fg * creg[i] + ig * gg;
                    hv = og * tanh_f(cn);
                } else if (a.mode == 1) {
                    // GRU on gate slots r, z, n (the fourth is empty): G holds
                    // x W_ih^T + b_ih + (b_hr, b_hz, 0); b_hn joins the hidden term
                    const float rg = sigmoid_f(sum.x + pre[0]);
                    const float zg = sigmoid_f(sum.y + pre[1]);
                    const float ng = tanh_f(pre[2] + rg * (sum.z + bhn[i]));
                    hv = (1.f - zg) * ng + zg * hreg[i];
                } else {
                    // plain RNN on the first gate slot
                    const float v = sum.x + pre[0];
                    hv = a.mode == 2 ? tanh_f(v) : fmaxf(v, 0.f);
                }
                if (t >= clen[i]) {  // padded step of this row: keep the state
                    cn = creg[i];
                    hv = hreg[i];
                }
                if (a.acts) {  // training: the activations the backward pass needs
                    float *ap = a.acts + (((size_t)t * B + b0 + cm[i]) * D + d) * 5 * H + j0 + cu[i];
                    ap[0] = ig;
                    ap[(size_t)H] = fg;
                    ap[(size_t)2 * H] = gg;
                    ap[(size_t)3 * H] = og;
                    ap[(size_t)4 * H] = cn;
                }
                creg[i] = cn;
                hreg[i] = hv;
                hs = DT::from_f(hv);
            }
            // word of (team row m, k) in the consumers' order:
            // ((tile * kch + chunk) * 64 + lane) * 4 + e, lane = 16 * g + m % 16
            const int m = cm[i], jj = j0 + cu[i];
            if constexpr (WIDE) {
                // one word per unit: lane 16 g + m % 16 reads units 8 g .. 8 g + 7 of its chunk
                if (publish && cv[i]) {
                    const int c = jj >> 5, g = (jj >> 3) & 3, e = jj & 7;
                    xcstore(xo + ((size_t)((m >> 4) * kch + c) * 64 + 16 * g + (m & 15)) * 8 + e,
                            xc_word_wide((uint16_t)hs, tb_out));
                }
            } else if constexpr (BF) {
                // units jj (even) and jj + 1 share a word; the even lane stores it
                const uint32_t mine_bits = (uint32_t)(uint16_t)hs;
                const uint32_t nb_bits = (uint32_t)__shfl_xor((int)mine_bits, 1);
                if (publish && cv[i] && (cu[i] & 1) == 0) {
                    const int c = jj >> 5, g = (jj >> 3) & 3, e = (jj >> 1) & 3;
                    const uint32_t hi = cu[i] + 1 < units ? nb_bits : 0u;
                    xcstore(xo + ((size_t)((m >> 4) * kch + c) * 64 + 16 * g + (m & 15)) * 4 + e,
                            xc_word_pair((uint16_t)mine_bits, (uint16_t)hi, tb_out));
                }
            } else if (publish && cv[i]) {
                const int c = jj >> 4, g = (jj >> 2) & 3, e = jj & 3;
                xcstore(xo + ((size_t)((m >> 4) * kch + c) * 64 + 16 * g + (m & 15)) * 4 + e,
                        xc_word_f32(__float_as_uint(hv), tb_out));
            }
            if (cv[i]) {
                const int bb = b0 + m;
                static_cast<S *>(a.Y)[trow(t, bb, T, B, a.bfirst) * ldy + (size_t)d * H + jj] = t < clen[i] ? hs : (S)0;
                if (s == T - 1) {
                    const size_t si = ((size_t)d * B + bb) * H + jj;
                    if (a.hn) static_cast<S *>(a.hn)[si] = hs;
                    if (a.cn) a.cn[si] = creg[i];
                }
            }
        }
        if constexpr (FUSED) load_x(s + 2, xcur);
        else load_g(s + 2, gcur);
        if (a.part_bufs != 2) __syncthreads();  // partials are reused by the next step
        t_pub = wall_clock64();
        return true;
    };
    for (int s = a.s_begin; s < a.s_end; s += 2) {
        if (!step(s, gA, xA)) return;
        if (s + 1 < a.s_end && !step(s + 1, gB, xB)) return;
    }

    if (a.s_end < T) {
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            if (cv[i]) {
                const size_t si = ((size_t)d * B + b0 + cm[i]) * H + j0 + cu[i];
                a.cstate[si] = creg[i];
                if (keep_h) a.hstate[si] = hreg[i];
            }
    }
}

// The instance of k_rec for tile t: W_hh in registers (wreg) or LDS, the
// input projection fused (fused: needs wreg) or hoisted; nullptr when the
// tile has no such instance.
template <class DT, bool XW>
const void *rec_kernel_variant(RecTile t, bool wreg, bool fused) {
    if (fused) {
        if (!wreg) return nullptr;
#define LSTM_F_PTR(wk, mtw, nt)                                                                    \
    if (t.WK == wk && t.MTW == mtw && t.NT == nt)                                                  \
        return reinterpret_cast<const void *>(&k_rec<DT, wk, mtw, nt, 8, true, LSTM_FX_OF(nt), XW>);
        LSTM_REC_FUSED_TILES(LSTM_F_PTR)
#undef LSTM_F_PTR
        return nullptr;
    }
#define LSTM_T_PTR(wk, mtw, nt)                                                                    \
    if (t.WK == wk && t.MTW == mtw && t.NT == nt)                                                  \
        return wreg ? reinterpret_cast<const void *>(&k_rec<DT, wk, mtw, nt, (mtw >= 4 ? 2 : 8), true, 0, XW>) \
                    : reinterpret_cast<const void *>(&k_rec<DT, wk, mtw, nt, (mtw >= 4 ? 2 : 8), false, 0, XW>);
    LSTM_REC_TILES(LSTM_T_PTR)
#undef LSTM_T_PTR
    return nullptr;
}

}  // namespace lstm_amd
