// rec_wave.hip -- the layer wavefront: every layer of a unidirectional LSTM
// stack in one persistent launch, the layers' workgroups sharing the CUs.
//
// Layer k > 0 takes the output of layer k-1 at the same time step as its
// input ("Long Short-Term Memory (LSTM)" on warp-nn, the symbol list; the
// MXNet blog "LSTM Forward Computation", "Stack Multiple RNN Cells"), so
// layer k can run step t as soon as layer k-1 has produced h_t, instead of
// after layer k-1's whole sequence.  Each layer keeps the per-step structure
// of the per-layer recurrence: a team of P workgroups owns a group of at most
// 16 batch rows, workgroup p owns hidden units [pU, pU + U) and keeps the
// matching 4U gate rows of W_hh and W_ih in registers as matrix-core
// fragments (W_hh in registers, W_ih in LDS: two workgroups share a CU's
// registers), and h_t travels between workgroups as tagged 32-bit words
// (device.h).  Layer 0 multiplies x_t (from memory) by its W_ih slice; layer
// k > 0 multiplies layer k-1's h_t, read from that layer's exchange words.
// Both products share one accumulator with the h_{t-1} product of the same
// equation block, and both biases are added in the epilogue.
//
// Why the layers share CUs: one layer's step is bound by the latency of the
// h exchange (write, visibility across the chip, read), not by its
// matrix-core work.  With two workgroups per CU -- one of each of two layers
// -- a CU's matrix cores work on one layer's products while the other layer
// waits for its exchange, so the CUs' matrix-core time per step is that of
// both layers while the wall time per step stays close to one layer's.
//
// Exchange buffers: layer k < L-1 writes step t into slot t of its own T
// slots (every word written once per call, tag 1; the buffer starts at zero,
// tag 0), so a layer never waits for its consumer; the last layer alternates
// two parity slots with step-alternating tags, like the per-layer kernel.
#include "device.h"
#include "kernels.h"

namespace lstm_amd {

namespace {

constexpr int kWaveCB = 8;  // K chunks of W_hh (and of a layer's W_ih) per wave: K <= 4 waves x 8 chunks

constexpr int kWaveLag = 2;

// s_waitcnt operand: vmcnt(0), expcnt and lgkmcnt not waited for
constexpr int kWaitVmem0 = (7 << 4) | (15 << 8);  // paired layers: layer 1 runs step t in the slot of layer 0's step t + 2

// LPW layers per workgroup: 1 (a workgroup per layer and unit slice), or 2
// (a two-layer stack's unit slice of both layers in one 512-thread
// workgroup, stepping in lockstep slots: layer 1 kWaveLag steps behind).
template <class DT, int NT, int FX, int LPW>
__global__ __launch_bounds__(256 * LPW, LPW == 2 ? 1 : (NT <= 2 ? 2 : 1)) void k_rec_wave(WaveArgs a) {
    using S = typename DT::S;
    constexpr bool BF = sizeof(S) == 2;
    constexpr int XF = BF ? XF_PAIR : XF_F32;  // |h| <= 1 for the LSTM: the pair words are sound
    constexpr int CB = kWaveCB;
    constexpr int ROWS = 16;                    // one 16-row tile per team
    constexpr int NCOL = 16 * NT;
    constexpr int U = 4 * NT;
    constexpr int PSTR = NCOL + 4;
    constexpr int CELLS = ROWS * U;
    constexpr int EW = BF ? 2 : 1;  // K values per exchange word
    static_assert(CELLS <= 256, "one cell per thread");
    static_assert(FX >= CB, "a layer above the first multiplies CB chunks of its input per wave");
    static_assert(LPW == 1 || LPW == 2, "one or two layers per workgroup");
    __shared__ float part[LPW][4 * ROWS * PSTR];
    __shared__ int s_bad;
    extern __shared__ __align__(16) unsigned char smem[];

    // a layer's 256 threads: wave wk owns a quarter of K
    // (the layer of a wave is the same for all its lanes: said so, so that it
    // stays in scalar registers and everything derived from it is uniform)
    const int tid = threadIdx.x & 255, lid = LPW == 2 ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 8)) : 0;
    const int lane = tid & 63, wk = tid >> 6;
    // W_ih fragments of this workgroup's layer lid: [wave][FX chunks][NT][64 lanes]
    u32x4 *wxs = reinterpret_cast<u32x4 *>(smem) + (size_t)lid * 4 * FX * NT * 64;
    // workgroup -> (layer, team, unit slice)
    const int per_layer = a.NGB * a.P;
    const int l = LPW == 2 ? lid : (int)(blockIdx.x / per_layer);
    const int lb = LPW == 2 ? (int)blockIdx.x : (int)(blockIdx.x % per_layer);
    int team, p;
    if (a.map_xcd) {  // workgroup ids go round-robin over the 8 XCDs; a team keeps to 8 / NGB of them
        const int X = 8 / a.NGB;
        team = (lb & 7) / X;
        p = (lb >> 3) * X + (lb & 7) % X;
    } else {
        team = lb / a.P;
        p = lb % a.P;
    }
    const int H = a.H, B = a.B, T = a.T, L = a.L, kch = a.kch;
    const int j0 = p * U, units = min(U, H - j0);
    const bool last = l == L - 1;
    const int I = l == 0 ? a.I : H;                       // input width of this layer
    const int ncx = l == 0 ? a.ncx0 : min(CB, max(0, kch - wk * CB));  // input chunks of this wave
    const int cx0 = l == 0 ? wk * a.ncx0 : wk * CB;       // first input chunk of this wave

    // Resident fragments: W_hh chunks [wk*CB, wk*CB + CB) in registers and
    // W_ih chunks [cx0, cx0 + ncx) in LDS, gate rows interleaved (local column
    // 4u + q), zero past H, past the input width and for dead units.
    u32x4 wreg[CB][NT];
    auto wx = [&](int cx, int j) -> u32x4 & { return wxs[((wk * FX + cx) * NT + j) * 64 + lane]; };
    {
        const S *W = static_cast<const S *>(a.whh[l]);
        const S *Wi = static_cast<const S *>(a.wih[l]);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int n = j * 16 + (lane & 15), u = n >> 2, q = n & 3;
#pragma unroll
            for (int ci = 0; ci < CB; ++ci) {
                const int k = (wk * CB + ci) * DT::KC + (lane >> 4) * DT::PER16;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (u < units && k < H) v = load_frag<DT>(W + (size_t)(q * H + j0 + u) * H, k, H, a.vec != 0);
                wreg[ci][j] = v;
            }
#pragma unroll
            for (int cx = 0; cx < FX; ++cx) {
                const int k = (cx0 + cx) * DT::KC + (lane >> 4) * DT::PER16;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (cx < ncx && u < units && k < I) v = load_frag<DT>(Wi + (size_t)(q * H + j0 + u) * I, k, I, a.vec != 0);
                wx(cx, j) = v;
            }
        }
    }

    // this thread's cell: team row cm, unit cu; c stays in a register for all T
    const int b0 = team * a.BG, rows = min(a.BG, B - b0);
    const int cm = tid / U, cu = tid % U;
    const bool cv = tid < CELLS && cm < rows && cu < units;
    const bool row_ok = (lane & 15) < rows;
    float creg = cv && a.c0 ? a.c0[((size_t)l * B + b0 + cm) * H + j0 + cu] : 0.f;
    float bias[4];
    {
        const S *bi = static_cast<const S *>(a.b_ih[l]), *bh = static_cast<const S *>(a.b_hh[l]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = q * H + j0 + (cv ? cu : 0);
            bias[q] = bi ? DT::to_f(bi[r]) + DT::to_f(bh[r]) : 0.f;
        }
    }
    if (threadIdx.x == 0) s_bad = 0;

    const int mrow = lane & 15;                    // this lane's team row in the 16-row tile
    const int ksub = (lane >> 4) * DT::PER16;      // this lane's K offset inside a chunk
    const size_t region = (size_t)kch * 256;       // exchange words of one team and slot
    auto slot_words = [&](int layer, int step) -> uint32_t * {
        const int sl = layer == L - 1 ? (step & 1) : step;
        return a.xbuf[layer] + ((size_t)sl * a.NGB + team) * region;
    };
    // tag of layer `layer`'s write at step `step`
    auto tag_of = [&](int layer, int step) -> unsigned { return layer == L - 1 ? xc_tag(0u, step) : 1u; };
    // word offset (bytes) of this lane's fragment of chunk c in a team region
    auto frag_off = [&](int c) -> unsigned { return (unsigned)(((size_t)c * 64 + lane) * 16); };

    // The input operand of a step, FX fragments: layer 0's x_t, loaded one
    // step ahead from memory (the buffer resource spans the batch rows of one
    // time step; dead rows and chunks read zeros), or layer l-1's h_t from
    // its exchange words.
    u32x4 xin[FX];
    auto load_x = [&](int step) __attribute__((always_inline)) {
        const int st = step < T ? step : T - 1;
        const int tx = __builtin_amdgcn_readfirstlane(st);
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<S *>(static_cast<const S *>(a.x) + (size_t)tx * B * a.I), (short)0,
            (int)((size_t)B * a.I * sizeof(S)), 0x00020000);
#pragma unroll
        for (int cx = 0; cx < FX; ++cx) {
            const int k = (cx0 + cx) * DT::KC + ksub;
            const bool ok = cx < ncx && row_ok && k < a.I;
            xin[cx] = __builtin_amdgcn_raw_buffer_load_b128(
                r, ok ? (int)(((size_t)(b0 + mrow) * a.I + k) * sizeof(S)) : 0x7FFFFFF0, 0, 0);
        }
    };
    if (l == 0) load_x(0);
    __syncthreads();

    long long t_pub = 0;
    // Exchange fragments: this lane's 16 bytes of chunks c0 .. c0 + CB of a
    // team region (live chunks below climit).  issue_words sends the loads;
    // wait_words checks their tags and re-reads until all carry tag tb, then
    // strips the tags (false: a wait gave up).
    auto nlive = [&](int c0, int climit, int ci) -> int {  // live words of fragment ci (recomputed: registers are scarce)
        const int c = c0 + ci, rem = H - c * DT::KC - ksub;
        return (!row_ok || c >= climit || rem <= 0) ? 0 : min(4, (rem + EW - 1) / EW);
    };
    // a fragment with no live word is read out of range: zeros, no memory access
    auto word_off = [&](int c0, int climit, int ci) -> unsigned {
        return nlive(c0, climit, ci) > 0 ? frag_off(c0 + ci) : 0x7FFFFFF0u;
    };
    auto issue_words = [&](const uint32_t *src, int c0, int climit, u32x4 (&frag)[CB]) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t xr = xcrsrc(src, (unsigned)(region * 4));
#pragma unroll
        for (int ci = 0; ci < CB; ++ci) frag[ci] = xload2(xr, word_off(c0, climit, ci));
    };
    // Whether every word of this wave's fragments of chunks c0 .. c0 + CB is
    // live (all 16 team rows, every chunk inside climit and H): wave-uniform,
    // and then no word needs settling, which keeps the per-word lane masks
    // (loop-invariant, spilled from scalar registers) off the step's path.
    auto all_live = [&](int c0, int climit) -> bool {
        return rows == ROWS && c0 + CB <= climit && (c0 + CB) * DT::KC <= H;
    };
    const bool live_x = l > 0 && all_live(cx0, kch), live_h = all_live(wk * CB, kch);
    auto wait_words = [&](const uint32_t *src, int c0, int climit, unsigned tb, bool live, u32x4 (&frag)[CB])
        __attribute__((always_inline)) -> bool {
        const __amdgpu_buffer_rsrc_t xr = xcrsrc(src, (unsigned)(region * 4));
        const unsigned tpat = tb << xc_shift(XF);
        auto settle = [&](int ci) __attribute__((always_inline)) {  // a dead word counts as current; its value meets zero W rows
            const int nl = nlive(c0, climit, ci);
            if (nl < 1) frag[ci].x = tpat;
            if (nl < 2) frag[ci].y = tpat;
            if (nl < 3) frag[ci].z = tpat;
            if (nl < 4) frag[ci].w = tpat;
        };
        // (short-circuit form: the branch-free one of the other kernels raises
        // the register count past two workgroups per CU here, and spills)
        bool mine = true;
#pragma unroll
        for (int ci = 0; ci < CB; ++ci) {
            if (!live) settle(ci);
            mine = mine && xc_ok<XF>(frag[ci], tb);
        }
        if (!__all(mine)) {
            unsigned spins = 0;
            const long long t0 = wall_clock64();
            do {
                if ((++spins & 31u) == 0) {
                    const unsigned st = __builtin_amdgcn_readfirstlane(
                        __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                    if (st != 0u) return false;
                    if (wall_clock64() - t0 > a.timeout_ticks) {
                        if (lane == 0) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        return false;
                    }
                }
                for (int z = 0; z < a.poll_sleep; ++z) __builtin_amdgcn_s_sleep(1);
                // Re-read every fragment, all issued before any is waited for.
                // A fragment already current reads the same words again: its
                // location is next written two steps later, which cannot
                // happen before this workgroup publishes its next step.
#pragma unroll
                for (int ci = 0; ci < CB; ++ci) frag[ci] = xload2(xr, word_off(c0, climit, ci));
                mine = true;
#pragma unroll
                for (int ci = 0; ci < CB; ++ci) {
                    if (!live) settle(ci);
                    mine = mine && xc_ok<XF>(frag[ci], tb);
                }
            } while (!__all(mine));
        }
        if constexpr (XF == XF_PAIR) {
#pragma unroll
            for (int ci = 0; ci < CB; ++ci)
                frag[ci] = u32x4{xc_pair_value(frag[ci].x), xc_pair_value(frag[ci].y), xc_pair_value(frag[ci].z),
                                 xc_pair_value(frag[ci].w)};
        }
        return true;
    };

    if (l > 0) issue_words(slot_words(l - 1, 0), cx0, kch, xin);  // step 0's input (checked in the step)
    // Step 0's input has returned before the loop, as every later step's has
    // at the bottom of the one before it (see below): the top of the step then
    // carries no wait for memory operations.
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);

    if constexpr (LPW == 2) {
        // Paired layers, three phases a slot, so that the two layers' critical
        // sections (h wait, recurrent product, epilogue, publication) never
        // compete for the matrix pipes: layer 0 runs its recurrent product in
        // phase 0, its epilogue in phase 1 and its next step's input product in
        // phase 2; layer 1 (kWaveLag steps behind, so that its input, layer 0's
        // h_t, is at least a slot old) its input product in phase 0, its
        // recurrent product in phase 1 and its epilogue in phase 2.  Each
        // layer's h is then published a phase or two before the team reads it.
        f32x4 acc[NT];
        long long t_pub2 = 0;
        // acc = x_s W_ih^T (x_s: layer 0's input, or layer 0's h_s for layer 1);
        // the next step's input is requested behind it
        auto input_task = [&](int st) __attribute__((always_inline)) -> bool {
            bool ok = true;
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (l > 0) ok = wait_words(slot_words(l - 1, st), cx0, kch, 1u, live_x, xin);
            if (ok) {
                u32x4 wcur[NT], wnext[NT];
#pragma unroll
                for (int j = 0; j < NT; ++j) wcur[j] = wx(0, j);
#pragma unroll
                for (int cx = 0; cx < FX; ++cx) {
                    if (cx < ncx) {
                        if (cx + 1 < FX)
#pragma unroll
                            for (int j = 0; j < NT; ++j) wnext[j] = wx(cx + 1, j);
#pragma unroll
                        for (int j = 0; j < NT; ++j) acc[j] = mma_chunk(DT{}, acc[j], xin[cx], wcur[j]);
#pragma unroll
                        for (int j = 0; j < NT; ++j) wcur[j] = wnext[j];
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (l == 0) load_x(st + 1);
            else if (st + 1 < T) issue_words(slot_words(l - 1, st + 1), cx0, kch, xin);
            return ok;
        };
        // acc += h_{s-1} W_hh^T at raised priority; the four K quarters' sums to LDS
        auto crit_task = [&](int st) __attribute__((always_inline)) -> bool {
            __builtin_amdgcn_s_setprio(2);
            bool ok = true;
            u32x4 hf[CB];
            if (st > 0) {
                if (a.pace > 0)
                    while (wall_clock64() - t_pub2 < a.pace) __builtin_amdgcn_s_sleep(1);
                issue_words(slot_words(l, st - 1), wk * CB, kch, hf);
                ok = wait_words(slot_words(l, st - 1), wk * CB, kch, tag_of(l, st - 1), live_h, hf);
            } else if (a.h0) {
                const S *hs = static_cast<const S *>(a.h0) + (size_t)l * B * H;
#pragma unroll
                for (int ci = 0; ci < CB; ++ci) {
                    const int k = (wk * CB + ci) * DT::KC + ksub;
                    hf[ci] = (row_ok && k < H) ? load_frag<DT>(hs + (size_t)(b0 + mrow) * H, k, H, a.vec != 0)
                                               : u32x4{0u, 0u, 0u, 0u};
                }
            }
            if (ok && (st > 0 || a.h0))
#pragma unroll
                for (int ci = 0; ci < CB; ++ci)
#pragma unroll
                    for (int j = 0; j < NT; ++j) acc[j] = mma_chunk(DT{}, acc[j], hf[ci], wreg[ci][j]);
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    part[lid][(wk * ROWS + 4 * (lane >> 4) + v) * PSTR + j * 16 + (lane & 15)] = acc[j][v];
            return ok;
        };
        // gates, cell update, h_t (warp-nn equation block), publication
        auto epi_task = [&](int st) __attribute__((always_inline)) {
            // every load of this wave has returned (its h wait drained them):
            // said so that the stores below are never waited for with the
            // next input
            __builtin_amdgcn_s_waitcnt(kWaitVmem0);
            float hv = 0.f;
            S hsv = (S)0;
            if (cv) {
                const f32x4 sum = lds_sum_f32x4<4>(&part[lid][cm * PSTR + 4 * cu], ROWS * PSTR);
                const float ig = sigmoid_f(sum.x + bias[0]);
                const float fg = sigmoid_f(sum.y + bias[1]);
                const float gg = tanh_f(sum.z + bias[2]);
                const float og = sigmoid_f(sum.w + bias[3]);
                creg = fg * creg + ig * gg;
                hv = og * tanh_f(creg);
                hsv = DT::from_f(hv);
            }
            const bool publish = !last || st + 1 < T;
            uint32_t *xo = slot_words(l, st);
            const unsigned tb_out = tag_of(l, st);
            const int jj = j0 + cu;
            if constexpr (BF) {
                const uint32_t mine_bits = (uint32_t)(uint16_t)hsv;
                const uint32_t nb_bits = (uint32_t)__shfl_xor((int)mine_bits, 1);
                if (publish && cv && (cu & 1) == 0) {
                    const int ch = jj >> 5, g = (jj >> 3) & 3, e = (jj >> 1) & 3;
                    const uint32_t hi = cu + 1 < units ? nb_bits : 0u;
                    xcstore(xo + ((size_t)ch * 64 + 16 * g + cm) * 4 + e,
                            xc_word_pair((uint16_t)mine_bits, (uint16_t)hi, tb_out));
                }
            } else if (publish && cv) {
                const int ch = jj >> 4, g = (jj >> 2) & 3, e = jj & 3;
                xcstore(xo + ((size_t)ch * 64 + 16 * g + cm) * 4 + e, xc_word_f32(__float_as_uint(hv), tb_out));
            }
            if (cv) {
                if (last) static_cast<S *>(a.Y)[((size_t)st * B + b0 + cm) * H + jj] = hsv;
                if (st == T - 1) {
                    const size_t si = ((size_t)l * B + b0 + cm) * H + jj;
                    if (a.hn) static_cast<S *>(a.hn)[si] = hsv;
                    if (a.cn) a.cn[si] = creg;
                }
            }
            t_pub2 = wall_clock64();
            __builtin_amdgcn_s_setprio(0);
        };

        if (l == 0) input_task(0);  // layer 0's first input product, ahead of the first slot
        const int nslots2 = T + kWaveLag;
        for (int sg = 0; sg < nslots2; ++sg) {
            const int st = sg - kWaveLag * l;
            const bool act = st >= 0 && st < T;
            bool ok = true;
            // phase 0: layer 0 critical, layer 1 input
            if (act) ok = l == 0 ? crit_task(st) : input_task(st);
            if (!ok) s_bad = 1;
            __syncthreads();
            if (s_bad) return;  // a wait gave up: leave (every workgroup drains the same way)
            // phase 1: layer 0 epilogue, layer 1 critical
            if (act) {
                if (l == 0) epi_task(st);
                else ok = crit_task(st);
            }
            if (!ok) s_bad = 1;
            __syncthreads();
            if (s_bad) return;
            // phase 2: layer 0 next input, layer 1 epilogue
            if (l == 0) {
                if (act && st + 1 < T) input_task(st + 1);
            } else if (act) {
                epi_task(st);
            }
            __syncthreads();  // the partial sums are reused in the next slot
        }
        return;
    }

    // slots: one step of every layer (paired layers: layer l at step sg - l kWaveLag,
    // idle before its first and after its last step but at every barrier)
    const int nslots = LPW == 2 ? T + kWaveLag * (L - 1) : T;
    for (int sg = 0; sg < nslots; ++sg) {
        const int s = LPW == 2 ? sg - kWaveLag * l : sg;
        const bool act = s >= 0 && s < T;
        bool wave_ok = true;
        f32x4 acc[NT];
        if (act) {
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

        // The input product first: x_t (layer 0) or layer l-1's h_t, both
        // read a step ahead (below).  Layer l-1's words are usually current
        // by now, since the layer below runs ahead; they are checked here and
        // re-read if not.  The W_ih fragments come from LDS one chunk ahead
        // of the products (the scheduling barriers keep the compiler from
        // fetching them all at once: registers are scarce with two
        // workgroups per CU).  The product also gives the others' h_{t-1}
        // time to arrive: their reads are issued after it (issued before it,
        // they reached memory ahead of the data and the step got slower).
        const uint32_t *xsrc = l > 0 ? slot_words(l - 1, s) : nullptr;
        if (l > 0) wave_ok = wait_words(xsrc, cx0, kch, 1u, live_x, xin);
        if (wave_ok) {
            u32x4 wcur[NT], wnext[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) wcur[j] = wx(0, j);
#pragma unroll
            for (int cx = 0; cx < FX; ++cx) {
                if (cx < ncx) {
                    if (cx + 1 < FX)
#pragma unroll
                        for (int j = 0; j < NT; ++j) wnext[j] = wx(cx + 1, j);
#pragma unroll
                    for (int j = 0; j < NT; ++j) acc[j] = mma_chunk(DT{}, acc[j], xin[cx], wcur[j]);
#pragma unroll
                    for (int j = 0; j < NT; ++j) wcur[j] = wnext[j];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // consumed: fetch the next step's input while this one runs
        if (l == 0) load_x(s + 1);
        else if (s + 1 < T) issue_words(slot_words(l - 1, s + 1), cx0, kch, xin);

        // From here to the publication of h_t the wave is on its layer's
        // critical path (every workgroup of the team waits for h_t): it takes
        // the matrix cores ahead of the other layer's input product, which
        // can run at any time before that layer's own h arrives.
        __builtin_amdgcn_s_setprio(2);

        // The hidden product: h_{t-1} (h0 at the first step), read once the
        // pace has passed since this workgroup's last publication.
        u32x4 hf[CB];
        const uint32_t *hsrc = s > 0 ? slot_words(l, s - 1) : nullptr;
        if (s > 0) {
            if (a.pace > 0)
                while (wall_clock64() - t_pub < a.pace) __builtin_amdgcn_s_sleep(1);
            issue_words(hsrc, wk * CB, kch, hf);
            if (wave_ok) wave_ok = wait_words(hsrc, wk * CB, kch, tag_of(l, s - 1), live_h, hf);
        } else if (a.h0) {  // plain loads of h0 (NULL: nothing to multiply)
            const S *hs = static_cast<const S *>(a.h0) + (size_t)l * B * H;
#pragma unroll
            for (int ci = 0; ci < CB; ++ci) {
                const int k = (wk * CB + ci) * DT::KC + ksub;
                hf[ci] = (row_ok && k < H) ? load_frag<DT>(hs + (size_t)(b0 + mrow) * H, k, H, a.vec != 0)
                                           : u32x4{0u, 0u, 0u, 0u};
            }
        }
        if (wave_ok && (s > 0 || a.h0))
#pragma unroll
            for (int ci = 0; ci < CB; ++ci)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[j] = mma_chunk(DT{}, acc[j], hf[ci], wreg[ci][j]);

        // partial sums of the four K quarters meet in LDS
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) part[lid][(wk * ROWS + 4 * (lane >> 4) + v) * PSTR + j * 16 + (lane & 15)] = acc[j][v];
        }  // act
        if (!wave_ok) s_bad = 1;
        // Every load of this wave has returned here on the usual path (the h
        // wait drained them); saying so on every path keeps the compiler from
        // waiting for the publication stores below at the top of the next
        // step, where it would otherwise wait for the prefetched input.
        __builtin_amdgcn_s_waitcnt(kWaitVmem0);
        __syncthreads();
        // The drain flag is read with the partial sums, in the same LDS round
        // trip, and tested once they are in.
        const int bad = s_bad;
        f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
        if (act && cv) sum = lds_sum_f32x4<4>(&part[lid][cm * PSTR + 4 * cu], ROWS * PSTR);
        if (bad) return;  // a wait gave up: leave (every workgroup drains the same way)
        if (act) {

        // gates, cell update, h_t (warp-nn equation block)
        float hv = 0.f;
        S hs = (S)0;
        if (cv) {
            const float ig = sigmoid_f(sum.x + bias[0]);
            const float fg = sigmoid_f(sum.y + bias[1]);
            const float gg = tanh_f(sum.z + bias[2]);
            const float og = sigmoid_f(sum.w + bias[3]);
            creg = fg * creg + ig * gg;
            hv = og * tanh_f(creg);
            hs = DT::from_f(hv);
        }
        // publish h_t in the consumers' fragment order (words of team row m, unit jj:
        // ((chunk * 64 + 16 g + m) * 4 + e)); the last layer's final step has no consumer
        const bool publish = !last || s + 1 < T;
        uint32_t *xo = slot_words(l, s);
        const unsigned tb_out = tag_of(l, s);
        const int jj = j0 + cu;
        if constexpr (BF) {
            // units jj (even) and jj + 1 share a word; the even lane stores it
            const uint32_t mine_bits = (uint32_t)(uint16_t)hs;
            const uint32_t nb_bits = (uint32_t)__shfl_xor((int)mine_bits, 1);
            if (publish && cv && (cu & 1) == 0) {
                const int ch = jj >> 5, g = (jj >> 3) & 3, e = (jj >> 1) & 3;
                const uint32_t hi = cu + 1 < units ? nb_bits : 0u;
                xcstore(xo + ((size_t)ch * 64 + 16 * g + cm) * 4 + e,
                        xc_word_pair((uint16_t)mine_bits, (uint16_t)hi, tb_out));
            }
        } else if (publish && cv) {
            const int ch = jj >> 4, g = (jj >> 2) & 3, e = jj & 3;
            xcstore(xo + ((size_t)ch * 64 + 16 * g + cm) * 4 + e, xc_word_f32(__float_as_uint(hv), tb_out));
        }
        if (cv) {
            if (last) static_cast<S *>(a.Y)[((size_t)s * B + b0 + cm) * H + jj] = hs;
            if (s == T - 1) {
                const size_t si = ((size_t)l * B + b0 + cm) * H + jj;
                if (a.hn) static_cast<S *>(a.hn)[si] = hs;
                if (a.cn) a.cn[si] = creg;
            }
        }
        }  // act
        __syncthreads();  // the partial sums are reused by the next step
        t_pub = wall_clock64();
        __builtin_amdgcn_s_setprio(0);
    }
}

// Paired layers only with NT <= 2: at NT = 4 two waves per SIMD do not fit
// the registers.
template <class DT>
const void *wave_kernel_ptr(int nt, int lpw) {
    if (nt == 1) return lpw == 2 ? reinterpret_cast<const void *>(&k_rec_wave<DT, 1, kWaveCB, 2>)
                                 : reinterpret_cast<const void *>(&k_rec_wave<DT, 1, kWaveCB, 1>);
    if (nt == 2) return lpw == 2 ? reinterpret_cast<const void *>(&k_rec_wave<DT, 2, kWaveCB, 2>)
                                 : reinterpret_cast<const void *>(&k_rec_wave<DT, 2, kWaveCB, 1>);
    if (nt == 4 && lpw == 1) return reinterpret_cast<const void *>(&k_rec_wave<DT, 4, kWaveCB, 1>);
    return nullptr;
}

const void *wave_kernel(int nt, int dtype, int lpw) {
    return dtype == DT_BF16 ? wave_kernel_ptr<BF16>(nt, lpw) : wave_kernel_ptr<F32>(nt, lpw);
}

}  // namespace

bool wave_shape_ok(int H, int I, int dtype, int *ncx0) {
    const int kc = dtype == DT_BF16 ? 32 : 16, per16 = dtype == DT_BF16 ? 8 : 4;
    const int kch = (H + kc - 1) / kc, kchi = (I + kc - 1) / kc;
    *ncx0 = (kchi + 3) / 4;
    // rows of whole 16-byte fragments (x and the weights are read 16 bytes at a time)
    return kch <= 4 * kWaveCB && *ncx0 <= kWaveCB && H % per16 == 0 && I % per16 == 0;
}

// dynamic LDS of k_rec_wave: the W_ih fragments of four waves per layer
static size_t wave_smem(int nt, int lpw) { return (size_t)lpw * 4 * kWaveCB * nt * 64 * 16; }

hipError_t wave_max_coresident(int nt, int dtype, int lpw, int *blocks_per_cu) {
    const void *fn = wave_kernel(nt, dtype, lpw);
    if (!fn) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)wave_smem(nt, lpw));
    if (e != hipSuccess) return e;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, 256 * lpw, wave_smem(nt, lpw));
}

hipError_t launch_wave(const WaveArgs &a, int nt, int dtype, int lpw, hipStream_t s) {
    const void *fn = wave_kernel(nt, dtype, lpw);
    if (!fn) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)wave_smem(nt, lpw));
    if (e != hipSuccess) return e;
    dim3 grid((lpw == 2 ? 1 : a.L) * a.NGB * a.P), block(256 * lpw);
    WaveArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchCooperativeKernel(fn, grid, block, args, (unsigned)wave_smem(nt, lpw), s);
}

}  // namespace lstm_amd
