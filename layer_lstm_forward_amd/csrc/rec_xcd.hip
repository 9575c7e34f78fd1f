// rec_xcd.hip -- the recurrence of one layer for small batches (at most 16
// rows), each direction's workgroups on a single XCD.
//
// The recurrence's step is bound by the h exchange between workgroups, and an
// exchange among the CUs of one XCD goes through that XCD's L2: measured on
// MI355X, an all-to-all round of tagged words takes about 0.9 us among 32
// workgroups of one XCD against 1.5 us or more across XCDs.  With B <= 16 the
// matrix-core work of a step is small (W_hh times one 16-row tile), so the
// whole of a direction's W_hh is held by the 32 CUs of one XCD: workgroup p
// owns hidden units [32p, 32p + 32), keeps their 128 gate rows of W_hh in
// registers across its eight waves (each wave an eighth of K), and the step's gate pre-activations are S = h_{t-1} W_hh^T (the warp-nn
// "Long Short-Term Memory (LSTM)" equation block) plus the hoisted input
// projection G[t] (both biases included).  The gates, the cell update and
// h_t are fused into the step, c stays in registers for all T, and h_t goes
// to the other workgroups as tagged words (device.h).  Direction d runs on XCD
// d; the other XCDs' workgroups of the launch leave at once.
#include "device.h"
#include "kernels.h"

namespace lstm_amd {

namespace {

constexpr int kXcdWaves = 8;   // waves per workgroup, each an eighth of K
constexpr int kXcdCPW = 4;     // K chunks per wave: K <= 8 x 4 chunks
constexpr int kXcdUnits = 32;  // hidden units per workgroup
constexpr int kXcdNT = kXcdUnits / 4;  // 16-column tiles of gate rows

template <class DT>
__global__ __launch_bounds__(512) void k_rec_xcd(RecArgs a) {
    using S = typename DT::S;
    constexpr bool BF = sizeof(S) == 2;
    constexpr int XF = BF ? XF_PAIR : XF_F32;  // |h| <= 1 for the LSTM: the pair words are sound
    constexpr int CPW = kXcdCPW, NT = kXcdNT, U = kXcdUnits, ROWS = 16;
    constexpr int NCOL = 16 * NT, PSTR = NCOL + 4;
    constexpr int EW = BF ? 2 : 1;
    __shared__ float part[kXcdWaves * ROWS * PSTR];
    __shared__ int s_bad;

    // workgroup ids go round-robin over the 8 XCDs: XCD d (id % 8) runs
    // direction d, its workgroups id / 8 = p own the unit slices
    const int xcd = blockIdx.x & 7, p = blockIdx.x >> 3;
    const int D = a.D, H = a.H, B = a.B, T = a.T, kch = a.kch;
    if (xcd >= D || p >= a.P) return;  // not a workgroup of this launch's teams
    const int d = xcd;
    const int tid = threadIdx.x, lane = tid & 63, wk = tid >> 6;
    const int j0 = p * U, units = min(U, H - j0);
    const int mrow = lane & 15, ksub = (lane >> 4) * DT::PER16;
    const bool row_ok = mrow < B;
    const size_t ldy = (size_t)D * H, ldg = (size_t)D * 4 * H;

    // W_hh fragments of this wave's K chunks [wk*CPW, wk*CPW + CPW), gate rows
    // interleaved (local column 4u + q), zero past H and for dead units
    u32x4 wreg[CPW][NT];
    {
        const S *W = static_cast<const S *>(a.whh[d]);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int n = j * 16 + (lane & 15), u = n >> 2, q = n & 3;
#pragma unroll
            for (int ci = 0; ci < CPW; ++ci) {
                const int k = (wk * CPW + ci) * DT::KC + ksub;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (u < units && k < H) v = load_frag<DT>(W + (size_t)(q * H + j0 + u) * H, k, H, a.vec != 0);
                wreg[ci][j] = v;
            }
        }
    }

    // this thread's cell: batch row cm, unit cu (512 threads = 16 rows x 32 units)
    const int cm = tid / U, cu = tid % U;
    const bool cv = cm < B && cu < units;
    const size_t si = ((size_t)d * B + (cv ? cm : 0)) * H + j0 + (cv ? cu : 0);
    float creg = cv && a.c0 ? a.c0[si] : 0.f;
    // G[t] of this cell, loaded one step ahead (a clamped valid address when dead)
    auto load_g = [&](int s, float (&g)[4]) {
        const int t = d == 0 ? min(s, T - 1) : T - 1 - min(s, T - 1);
        const float *gp = a.G + ((size_t)t * B + (cv ? cm : 0)) * ldg + (size_t)d * 4 * H + j0 + (cv ? cu : 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) g[q] = gp[(size_t)q * H];
    };
    float gnext[4];
    load_g(0, gnext);
    if (tid == 0) s_bad = 0;
    __syncthreads();

    const size_t region = (size_t)kch * 256;  // exchange words of the team
    uint32_t *const xb32 = reinterpret_cast<uint32_t *>(a.xbuf);
    auto xslot = [&](int s) { return xb32 + ((size_t)(s & 1) * D + d) * region; };
    auto nlive = [&](int ci) -> int {  // live words of this lane's fragment of chunk wk*CPW + ci
        const int c = wk * CPW + ci, rem = H - c * DT::KC - ksub;
        return (!row_ok || c >= kch || rem <= 0) ? 0 : min(4, (rem + EW - 1) / EW);
    };
    auto word_off = [&](int ci) -> unsigned {  // no live word: out of range (zeros, no memory access)
        return nlive(ci) > 0 ? (unsigned)((((size_t)(wk * CPW + ci)) * 64 + lane) * 16) : 0x7FFFFFF0u;
    };
    long long t_pub = 0;

    for (int s = 0; s < T; ++s) {
        const int t = d == 0 ? s : T - 1 - s;
        float g[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) g[q] = gnext[q];

        f32x4 acc[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        bool wave_ok = true;
        u32x4 hf[CPW];
        bool have_h = true;
        if (s == 0) {
            have_h = a.h0 != nullptr;
            if (have_h) {
                const S *hs = static_cast<const S *>(a.h0) + (size_t)d * B * H;
#pragma unroll
                for (int ci = 0; ci < CPW; ++ci) {
                    const int k = (wk * CPW + ci) * DT::KC + ksub;
                    hf[ci] = (row_ok && k < H) ? load_frag<DT>(hs + (size_t)mrow * H, k, H, a.vec != 0)
                                               : u32x4{0u, 0u, 0u, 0u};
                }
            }
        } else {
            // h_{t-1} from the exchange words of step s-1, once the pace has
            // passed since this workgroup's own publication
            const unsigned tb = xc_tag(a.xpar, s - 1);
            const __amdgpu_buffer_rsrc_t xr = xcrsrc(xslot(s - 1), (unsigned)(region * 4));
            if (a.pace > 0)
                while (wall_clock64() - t_pub < a.pace) __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int ci = 0; ci < CPW; ++ci) hf[ci] = xload2(xr, word_off(ci));
            const unsigned tpat = tb << xc_shift(XF);
            auto settle = [&](int ci) {  // a dead word counts as current; its value meets zero W rows
                const int nl = nlive(ci);
                if (nl < 1) hf[ci].x = tpat;
                if (nl < 2) hf[ci].y = tpat;
                if (nl < 3) hf[ci].z = tpat;
                if (nl < 4) hf[ci].w = tpat;
            };
            bool mine = true;
#pragma unroll
            for (int ci = 0; ci < CPW; ++ci) {
                settle(ci);
                mine = mine & xc_ok<XF>(hf[ci], tb);
            }
            if (!__all(mine)) {
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
                                __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            wave_ok = false;
                            break;
                        }
                    }
                    for (int z = 0; z < a.poll_sleep; ++z) __builtin_amdgcn_s_sleep(1);
                    // re-read every fragment (a current one reads the same words again:
                    // its location is next written two steps later)
#pragma unroll
                    for (int ci = 0; ci < CPW; ++ci) hf[ci] = xload2(xr, word_off(ci));
                    mine = true;
#pragma unroll
                    for (int ci = 0; ci < CPW; ++ci) {
                        settle(ci);
                        mine = mine & xc_ok<XF>(hf[ci], tb);
                    }
                } while (!__all(mine));
            }
            if constexpr (XF == XF_PAIR) {
#pragma unroll
                for (int ci = 0; ci < CPW; ++ci)
                    hf[ci] = u32x4{xc_pair_value(hf[ci].x), xc_pair_value(hf[ci].y), xc_pair_value(hf[ci].z),
                                   xc_pair_value(hf[ci].w)};
            }
        }
        // The next step's G is requested only now: vector-memory counters
        // complete in issue order, so loads issued before the h reads would
        // hold up the check of those reads until they too had returned
        // (G comes from HBM, h from the exchange, sooner).
        load_g(s + 1, gnext);
        if (wave_ok && have_h)
#pragma unroll
            for (int ci = 0; ci < CPW; ++ci)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[j] = mma_chunk(DT{}, acc[j], hf[ci], wreg[ci][j]);

        // the eight K slices' partial sums meet in LDS
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) part[(wk * ROWS + 4 * (lane >> 4) + v) * PSTR + j * 16 + (lane & 15)] = acc[j][v];
        if (!wave_ok) s_bad = 1;
        __syncthreads();
        if (s_bad) return;  // a wait gave up: leave (every workgroup drains the same way)

        // gates, cell update, h_t (warp-nn equation block)
        float hv = 0.f;
        S hs = (S)0;
        if (cv) {
            const float *pp = &part[cm * PSTR + 4 * cu];
            const f32x4 sum = lds_sum_f32x4<kXcdWaves>(pp, ROWS * PSTR);
            const float ig = sigmoid_f(sum.x + g[0]);
            const float fg = sigmoid_f(sum.y + g[1]);
            const float gg = tanh_f(sum.z + g[2]);
            const float og = sigmoid_f(sum.w + g[3]);
            creg = fg * creg + ig * gg;
            hv = og * tanh_f(creg);
            hs = DT::from_f(hv);
        }
        // publish h_t in the consumers' fragment order: word of row m, unit jj
        // at ((chunk * 64 + 16 g + m) * 4 + e)
        const bool publish = s + 1 < T;
        uint32_t *xo = xslot(s);
        const unsigned tb_out = xc_tag(a.xpar, s);
        const int jj = j0 + cu;
        if constexpr (BF) {
            // units jj (even) and jj + 1 share a word; the even lane stores it
            const uint32_t mine_bits = (uint32_t)(uint16_t)hs;
            const uint32_t nb_bits = (uint32_t)__shfl_xor((int)mine_bits, 1);
            if (publish && cv && (cu & 1) == 0) {
                const int ch = jj >> 5, gq = (jj >> 3) & 3, e = (jj >> 1) & 3;
                const uint32_t hi = cu + 1 < units ? nb_bits : 0u;
                xcstore(xo + ((size_t)ch * 64 + 16 * gq + cm) * 4 + e,
                        xc_word_pair((uint16_t)mine_bits, (uint16_t)hi, tb_out));
            }
        } else if (publish && cv) {
            const int ch = jj >> 4, gq = (jj >> 2) & 3, e = jj & 3;
            xcstore(xo + ((size_t)ch * 64 + 16 * gq + cm) * 4 + e, xc_word_f32(__float_as_uint(hv), tb_out));
        }
        if (cv) {
            static_cast<S *>(a.Y)[((size_t)t * B + cm) * ldy + (size_t)d * H + jj] = hs;
            if (s == T - 1) {
                if (a.hn) static_cast<S *>(a.hn)[si] = hs;
                if (a.cn) a.cn[si] = creg;
            }
        }
        __syncthreads();  // the partial sums are reused by the next step
        t_pub = wall_clock64();
    }
}

}  // namespace

bool xcd_shape_ok(int H, int B, int D, int dtype) {
    const int kc = dtype == DT_BF16 ? 32 : 16, per16 = dtype == DT_BF16 ? 8 : 4;
    const int kch = (H + kc - 1) / kc, P = (H + kXcdUnits - 1) / kXcdUnits;
    return B <= 16 && D <= 2 && kch <= kXcdWaves * kXcdCPW && P <= 32 && H % per16 == 0;
}

int xcd_workgroups(int H) { return (H + kXcdUnits - 1) / kXcdUnits; }

static const void *xcd_kernel(int dtype) {
    return dtype == DT_BF16 ? reinterpret_cast<const void *>(&k_rec_xcd<BF16>)
                            : reinterpret_cast<const void *>(&k_rec_xcd<F32>);
}

hipError_t xcd_max_coresident(int dtype, int *blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, xcd_kernel(dtype), 512, 0);
}

hipError_t launch_xcd(const RecArgs &a, int dtype, hipStream_t s) {
    // 8 workgroup ids per unit slice: id % 8 is the XCD, and only XCD d < D works
    dim3 grid(8 * a.P), block(512);
    RecArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchCooperativeKernel(xcd_kernel(dtype), grid, block, args, 0, s);
}

}  // namespace lstm_amd
