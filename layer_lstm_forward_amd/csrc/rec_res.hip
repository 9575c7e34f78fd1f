// rec_res.hip -- the recurrence of one layer for large batches whose W_hh
// does not fit on chip once per batch tile: W_hh held once across the chip.
//
// The step is S = h_{t-1} W_hh^T for B rows (the warp-nn "Long Short-Term
// Memory (LSTM)" equation block) plus the hoisted projection G[t], then the
// gates and the cell update.  At B = 256, H = 2048 the product is a
// 256 x 8192 x 2048 GEMM per step.  Streaming W_hh (32 MiB in bf16) through
// L2 every step bounds a per-step launch by that stream; here it is read
// once per launch instead.  Workgroup (m, n) owns batch rows [128m, 128m+128)
// and hidden units [16n, 16n+16): 64 gate rows of W_hh, which its four waves
// hold in registers, each a quarter of K (CPW chunks of 32: up to 256
// registers a wave, which the matrix cores read as their second operand
// straight from the accumulation registers).  A wave multiplies h_{t-1} over
// its K quarter for all of the workgroup's rows; the quarters' partial sums
// meet in LDS, and each wave then finishes the cells of one 16-row tile.  A
// step runs in two passes of 64 rows each, so that a pass's accumulators and
// loads in flight fit beside W_hh, and the rows of a pass are published
// before the next pass is computed: the pass that reads them comes a whole
// pass later.
//
// Every workgroup of a row block reads all of that block's h_{t-1} each
// step (512 KiB at H = 2048), so the step is bound by how fast the CUs read
// h from their L2.  h travels through a two-slot ring laid out in the
// consumers' fragment order: the 16 bytes lane l feeds the matrix core for
// row tile i and K chunk c sit at ((i * KC + c) * 64 + l) * 16 within the
// block's slot, so every load is 1 KiB contiguous (row-major fragments of y,
// 16 rows x 64 bytes a load, read at half that rate).  Words are the compact
// bf16 pair words of the other recurrent kernels (two adjacent units, one-bit
// step tag in bit 30: the LSTM's |h| <= 1 leaves it free), stored with
// device-scope atomic 32-bit stores and re-read with device-scope loads until
// their tag is current.  A slot is rewritten every two steps; a consumer can
// only see its previous write or the current one, because the producer's
// next write to it needs this consumer's own publication of the step in
// between.  y gets ordinary stores.  The ring is zeroed before the launch
// (tag 0).
//
// L2 warm-up: the producers' writes invalidate the lines in the other XCDs'
// L2s, and every workgroup of an XCD then wants the same fresh lines at once.
// While a pass ends, each workgroup loads its share of the block the next
// pass reads (the XCD's workgroups of the row block split it between them),
// so the next pass's loads find the lines in L2.
#include "device.h"
#include "kernels.h"

namespace lstm_amd {

namespace {

constexpr int kResUnits = 16;    // hidden units per workgroup (64 gate rows)
constexpr int kResRows = 128;    // batch rows per workgroup
constexpr int kResRTP = 4;       // 16-row tiles per pass: one per wave in the epilogue
constexpr int kResPasses = kResRows / (16 * kResRTP);
constexpr int kResTiles = kResRows / 16;
#ifndef RES_LA
#define RES_LA 2
#endif
constexpr int kResLA = RES_LA;               // chunks whose loads are in flight ahead of the one multiplied
constexpr unsigned kResOOR = 0x80000000u;    // a buffer offset past any resource: reads zero
constexpr int kResSC1 = 16;                  // cache policy of a device-scope load
// s_waitcnt operands: vmcnt <= 6 (expcnt, lgkmcnt not waited for); lgkmcnt = 0 only
constexpr int kWaitAllButNext = 6 | (7 << 4) | (15 << 8);
constexpr int kWaitLds = 15 | (7 << 4) | (3 << 14);
typedef __attribute__((address_space(3))) void lds_void_t;

template <int CPW>
__global__ __launch_bounds__(256, 1) void k_rec_res(RecArgs a) {
    using DT = BF16;
    using S = DT::S;
    constexpr int KC = 4 * CPW;  // K chunks of 32 in H
    // the chunk after whose loads the next pass's loads are issued: the last one loaded
    constexpr int kIssueAt = CPW - 1 - kResLA > 0 ? CPW - 1 - kResLA : 0;
    // partial sums of each pass: [pass][destination row tile][other wave][gate][lane]
    __shared__ f32x4 part[kResPasses][kResRTP][kResRTP - 1][4][64];
    // G of each wave's cells in each pass: [wave][pass][row of the tile][gate][unit]
    __shared__ __align__(16) float gsh[kResRTP][kResPasses][16][4][kResUnits];
    // landing area of the L2 warm-up loads (never read)
    __shared__ __align__(16) u32x4 warm[kResRTP][64];
    // each wave's h_t tile, to be read back by row
    __shared__ __align__(16) S hx[kResRTP][16][kResUnits];
    __shared__ int s_bad;

    const int D = a.D, H = a.H, B = a.B, T = a.T;
    const int NG = a.NGB, P = a.P;  // groups (row block, direction) and unit slices per group
    int grp, n;
    int xi, nx;  // this workgroup's index among the group's workgroups on its XCD, and their number
    {
        const int bid = blockIdx.x;
        if (a.map_xcd) {
            // workgroup ids go round-robin over the 8 XCDs: a group's slices
            // share XCDs, so the h rows they all read are fetched into those L2s
            const int per = 8 / NG;
            grp = (bid & 7) / per;
            n = (bid >> 3) * per + (bid & 7) % per;
            xi = bid >> 3;
            nx = P / per;
        } else {
            grp = bid / P;
            n = bid % P;
            xi = n;
            nx = P;
        }
    }
    if (grp >= NG || n >= P) return;
    const int d = grp % D, m = grp / D;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // this wave's K quarter
    const int b0 = m * kResRows, j0 = n * kResUnits;
    const int nrows = min(kResRows, B - b0);
    const int ksub = 8 * (lane >> 4), u = lane & 15;
    const size_t ldy = (size_t)D * H, ldg = (size_t)D * 4 * H;
    // ring: [slot 2][group NG][tile 8][chunk KC][lane 64] 16-byte fragments
    constexpr unsigned kSlotBytes = (unsigned)kResTiles * KC * 1024u;
    uint32_t *const ring = reinterpret_cast<uint32_t *>(a.xbuf);
    auto ring_block = [&](int slot) { return ring + ((size_t)slot * NG + grp) * (kSlotBytes / 4); };

    // W_hh fragments of this wave's K quarter: gate q, unit j0 + u (row q*H + j0 + u)
    u32x4 wreg[CPW][4];
    {
        const S *W = static_cast<const S *>(a.whh[d]);
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                wreg[c][q] = *reinterpret_cast<const u32x4 *>(W + (size_t)(q * H + j0 + u) * H + (w * CPW + c) * 32 + ksub);
    }

    // this wave's cells: in pass p, row tile p * kResRTP + w, rows 4 (lane / 16) + v, unit j0 + u
    auto cell_row = [&](int p, int v) { return 16 * (p * kResRTP + w) + 4 * (lane >> 4) + v; };
    float creg[kResPasses][4];
#pragma unroll
    for (int p = 0; p < kResPasses; ++p)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = cell_row(p, v);
            creg[p][v] = (a.c0 && row < nrows) ? a.c0[((size_t)d * B + b0 + row) * H + j0 + u] : 0.f;
        }
    if (tid == 0) s_bad = 0;
    __syncthreads();

    S *const y = static_cast<S *>(a.Y);
    S *const hn = static_cast<S *>(a.hn);
    // G of this wave's cells in pass p of step s (both biases included) goes
    // straight into LDS: four 1 KiB loads, rows 4r .. 4r + 3 of the tile,
    // lane l -> row 4r + l / 16, gate (l / 4) % 4, units 4 (l % 4) ..  Past
    // the last step the loads read nothing (an empty resource), so that every
    // pass issues the same number of them.
    auto load_g = [&](int s, int p) {
        const int t = d == 0 ? s : T - 1 - s;
        const int rt0 = 16 * (p * kResRTP + w);
        const int rows_here = s < T ? min(16, max(0, nrows - rt0)) : 0;
        const float *gbase = a.G + ((size_t)(s < T ? t : 0) * B + b0 + rt0) * ldg + (size_t)d * 4 * H + j0;
        const unsigned gbytes =
            rows_here > 0 ? (unsigned)((((size_t)rows_here - 1) * ldg + 3 * H + kResUnits) * 4) : 0u;
        const __amdgpu_buffer_rsrc_t gr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(gbase), (short)0, (int)gbytes, 0x00020000);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * r + (lane >> 4), q = (lane >> 2) & 3, sg = lane & 3;
            const unsigned go = (unsigned)(((size_t)row * ldg + (size_t)q * H + 4 * sg) * 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(gr, (lds_void_t *)&gsh[w][p][4 * r][0][0], 16, go, 0, 0, 0);
        }
    };
    // Warm this XCD's L2 with this workgroup's share of the ring block that
    // pass p of step s reads (its four row tiles, all KC chunks: 4 KC KiB,
    // split in 1 KiB pieces over the XCD's workgroups of the group, two a
    // wave).  The data land in a scratch LDS area nobody reads.
    auto warm_h = [&](int s, int p) {
        const bool on = s >= 1 && s < T;  // step 0 reads h0, not the ring
        const uint32_t *blk = ring_block(on ? (s - 1) & 1 : 0) + (size_t)p * kResRTP * KC * 256;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t *>(blk), (short)0, on ? (int)(kResRTP * KC * 1024) : 0, 0x00020000);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int piece = (j * kResRTP + w) * nx + xi;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)&warm[w][0], 16,
                                                     (unsigned)piece * 1024u + lane * 16u, 0, 0, 0);
        }
    };

    load_g(0, 0);
    for (int s = 0; s < T; ++s) {
        const int t = d == 0 ? s : T - 1 - s;
        // h_{t-1}: h0 at the first step (row-major, read once), else the ring slot
        // written at step s - 1
        const S *h0p = a.h0 ? static_cast<const S *>(a.h0) + ((size_t)d * B + b0) * H : nullptr;
        const bool from_h0 = s == 0;
        const bool have_h = !from_h0 || h0p;
        const unsigned tb = xc_tag(0u, s - 1);        // tag of the words written at step s - 1
        const unsigned tb_out = xc_tag(0u, s);        // tag of this step's words
        const __amdgpu_buffer_rsrc_t hr =
            from_h0 ? __builtin_amdgcn_make_buffer_rsrc(const_cast<S *>(h0p), (short)0,
                                                        h0p ? (int)((((size_t)nrows - 1) * H + H) * sizeof(S)) : 0,
                                                        0x00020000)
                    : __builtin_amdgcn_make_buffer_rsrc(ring_block((s - 1) & 1), (short)0, (int)kSlotBytes,
                                                        0x00020000);
        const __amdgpu_buffer_rsrc_t out_r =
            __builtin_amdgcn_make_buffer_rsrc(ring_block(s & 1), (short)0, (int)kSlotBytes, 0x00020000);

#pragma unroll
        for (int p = 0; p < kResPasses; ++p) {
            // the pass that follows this one: its G and its h block are fetched
            // while this pass's last chunks are multiplied (the block it reads
            // was published a pass ago)
            const int sn = p + 1 < kResPasses ? s : s + 1, pn = (p + 1) % kResPasses;
            auto issue_next = [&]() {
                load_g(sn, pn);
                warm_h(sn, pn);
            };
            f32x4 acc[kResRTP][4];
#pragma unroll
            for (int i = 0; i < kResRTP; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[i][q] = f32x4{0.f, 0.f, 0.f, 0.f};
            bool wave_ok = true;
            if (have_h) {
                // lane's 16 bytes of row tile i, chunk c: from the ring, a
                // contiguous 1 KiB fragment; from h0, a row-major fragment (rows
                // past B: out of range, zeros)
                unsigned vo[kResRTP];
                int so, cstride;
                if (from_h0) {
#pragma unroll
                    for (int i = 0; i < kResRTP; ++i) {
                        const int row = 16 * (p * kResRTP + i) + (lane & 15);
                        vo[i] = row < nrows ? (unsigned)(((size_t)row * H + ksub) * sizeof(S)) : kResOOR;
                    }
                    so = w * CPW * 64;
                    cstride = 64;
                } else {
#pragma unroll
                    for (int i = 0; i < kResRTP; ++i) vo[i] = (unsigned)((p * kResRTP + i) * KC * 1024 + lane * 16);
                    so = w * CPW * 1024;
                    cstride = 1024;
                }
                auto ld4 = [&](u32x4 (&f)[kResRTP], int c) {
#pragma unroll
                    for (int i = 0; i < kResRTP; ++i)
                        f[i] = __builtin_amdgcn_raw_buffer_load_b128(hr, (int)(vo[i] + c * cstride), so, kResSC1);
                };
                // every word of the four fragments carries the expected tag
                auto current = [&](const u32x4 (&f)[kResRTP]) {
                    bool ok = true;
#pragma unroll
                    for (int i = 0; i < kResRTP; ++i) ok = ok & xc_ok<XF_PAIR>(f[i], tb);
                    return from_h0 || ok;
                };
                u32x4 hf[kResLA + 1][kResRTP];
#pragma unroll
                for (int c = 0; c < kResLA && c < CPW; ++c) ld4(hf[c], c);
#pragma unroll
                for (int c = 0; c < CPW; ++c) {
                    if (c + kResLA < CPW) ld4(hf[(c + kResLA) % (kResLA + 1)], c + kResLA);
                    // after the pass's last h loads: no later wait of this pass
                    // waits for these (the counter is in issue order)
                    if (c == kIssueAt) issue_next();
                    u32x4(&f)[kResRTP] = hf[c % (kResLA + 1)];
                    if (!wave_ok) continue;
                    if (!__all(current(f))) {
                        // some producer of this chunk has not published yet: re-read the chunk
                        unsigned spins = 0;
                        const long long t0 = wall_clock64();
                        while (true) {
                            if ((++spins & 31u) == 0) {
                                const unsigned st = __builtin_amdgcn_readfirstlane(
                                    __hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                                if (st != 0u) {
                                    wave_ok = false;
                                    break;
                                }
                                if (wall_clock64() - t0 > a.timeout_ticks) {
                                    if (lane == 0)
                                        __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                    wave_ok = false;
                                    break;
                                }
                            }
                            for (int z = 0; z < a.poll_sleep; ++z) __builtin_amdgcn_s_sleep(1);
                            ld4(f, c);
                            if (__all(current(f))) break;
                        }
                        if (!wave_ok) continue;
                    }
                    if (!from_h0) {
#pragma unroll
                        for (int i = 0; i < kResRTP; ++i)
                            f[i] = u32x4{xc_pair_value(f[i].x), xc_pair_value(f[i].y), xc_pair_value(f[i].z),
                                         xc_pair_value(f[i].w)};
                    }
#pragma unroll
                    for (int i = 0; i < kResRTP; ++i)
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[i][q] = mma_chunk(DT{}, acc[i][q], f[i], wreg[c][q]);
                }
            }

            if (!have_h) issue_next();

            // the K quarters meet in LDS: each wave hands the other waves' row tiles over
#pragma unroll
            for (int i = 0; i < kResRTP; ++i)
                if (i != w) {
                    const int sl = w < i ? w : w - 1;
#pragma unroll
                    for (int q = 0; q < 4; ++q) part[p][i][sl][q][lane] = acc[i][q];
                }
            if (!wave_ok) s_bad = 1;
            // a barrier that waits only for this wave's LDS writes: the next
            // pass's loads stay in flight (a workgroup fence would wait for them,
            // since some of them write LDS)
            __builtin_amdgcn_s_waitcnt(kWaitLds);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            // the drain flag is read with the partial sums (one LDS round trip)
            const int bad = s_bad;
            f32x4 sum[4];
#pragma unroll
            for (int i = 0; i < kResRTP; ++i)
                if (i == w)
#pragma unroll
                    for (int q = 0; q < 4; ++q) sum[q] = acc[i][q];
#pragma unroll
            for (int sl = 0; sl < kResRTP - 1; ++sl)
#pragma unroll
                for (int q = 0; q < 4; ++q) sum[q] += part[p][w][sl][q][lane];
            if (bad) return;  // a wait gave up: leave (every workgroup drains the same way)

            // this wave's G loads of this pass are in LDS (it alone reads them):
            // all but the six newest loads (the next pass's) have completed
            __builtin_amdgcn_s_waitcnt(kWaitAllButNext);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            // gates, cell update, h_t (warp-nn equation block)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = cell_row(p, v);
                const float *gv = &gsh[w][p][4 * (lane >> 4) + v][0][u];
                const float ig = sigmoid_f(sum[0][v] + gv[0]);
                const float fg = sigmoid_f(sum[1][v] + gv[kResUnits]);
                const float gg = tanh_f(sum[2][v] + gv[2 * kResUnits]);
                const float og = sigmoid_f(sum[3][v] + gv[3 * kResUnits]);
                creg[p][v] = fg * creg[p][v] + ig * gg;
                const S hs = DT::from_f(og * tanh_f(creg[p][v]));
                hx[w][4 * (lane >> 4) + v][u] = hs;
                if (s == T - 1 && row < nrows) {
                    const size_t si = ((size_t)d * B + b0 + row) * H + j0 + u;
                    if (hn) hn[si] = hs;
                    if (a.cn) a.cn[si] = creg[p][v];
                }
            }
            // h_t of the wave's 16 x 16 cells, read back by row: lane l < 32
            // takes row l / 2, units 8 (l % 2) .. + 7 (16 bytes), which is one
            // lane's slot of a ring fragment and 16 contiguous bytes of y, so
            // each 128-byte line of the ring is written by one instruction.
            // (LDS operations of one wave complete in order.)
            if (lane < 32) {
                const int r = lane >> 1, half = lane & 1;
                const int row = 16 * (p * kResRTP + w) + r;
                const u32x4 hv = *reinterpret_cast<const u32x4 *>(&hx[w][r][8 * half]);
                const int jj = j0 + 8 * half;  // first unit of the 16 bytes
                if (s + 1 < T) {
                    // ring slot: fragment (tile, jj / 32), lane r + 16 ((jj % 32) / 8)
                    const int tile = p * kResRTP + w;
                    const unsigned off = (unsigned)(((tile * KC + jj / 32) * 64 + r + 16 * ((jj % 32) / 8)) * 16);
                    const u32x4 wv = {xc_word_pair((uint16_t)hv.x, (uint16_t)(hv.x >> 16), tb_out),
                                      xc_word_pair((uint16_t)hv.y, (uint16_t)(hv.y >> 16), tb_out),
                                      xc_word_pair((uint16_t)hv.z, (uint16_t)(hv.z >> 16), tb_out),
                                      xc_word_pair((uint16_t)hv.w, (uint16_t)(hv.w >> 16), tb_out)};
                    // a device-scope store: each 4-byte word lands whole
                    __builtin_amdgcn_raw_buffer_store_b128(wv, out_r, (int)off, 0, kResSC1);
                }
                if (row < nrows)
                    *reinterpret_cast<u32x4 *>(y + ((size_t)t * B + b0 + row) * ldy + (size_t)d * H + jj) = hv;
            }
        }
    }
}

// K chunks per wave of each instance: H = 128 CPW
constexpr int kResCPWs[] = {2, 4, 8, 12, 16};

const void *res_kernel(int H) {
    switch (H / 128) {
        case 2: return reinterpret_cast<const void *>(&k_rec_res<2>);
        case 4: return reinterpret_cast<const void *>(&k_rec_res<4>);
        case 8: return reinterpret_cast<const void *>(&k_rec_res<8>);
        case 12: return reinterpret_cast<const void *>(&k_rec_res<12>);
        case 16: return reinterpret_cast<const void *>(&k_rec_res<16>);
        default: return nullptr;
    }
}

}  // namespace

bool res_shape_ok(int H, int B, int D, int dtype, int cus, int *groups, int *slices, int *map_xcd) {
    if (dtype != DT_BF16 || H % 128 != 0 || B < 1 || D < 1 || D > 2) return false;
    bool listed = false;
    for (int c : kResCPWs) listed = listed || H == 128 * c;
    if (!listed) return false;
    const int g = ((B + kResRows - 1) / kResRows) * D, pn = H / kResUnits;
    if ((long long)g * pn > cus) return false;
    if (groups) *groups = g;
    if (slices) *slices = pn;
    if (map_xcd) *map_xcd = (8 % g == 0 && pn % (8 / g) == 0) ? 1 : 0;
    return true;
}

size_t res_ring_bytes(int H, int groups) {
    return (size_t)2 * groups * kResTiles * (H / 32) * 1024;
}

hipError_t res_max_coresident(int H, int *blocks_per_cu) {
    const void *k = res_kernel(H);
    if (!k) return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, k, 256, 0);
}

hipError_t launch_res(const RecArgs &a, hipStream_t s) {
    const void *k = res_kernel(a.H);
    if (!k) return hipErrorInvalidValue;
    dim3 grid(a.NGB * a.P), block(256);
    RecArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchCooperativeKernel(k, grid, block, args, 0, s);
}

}  // namespace lstm_amd
