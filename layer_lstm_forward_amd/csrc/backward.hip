// backward.hip -- gfx950 kernels of the LSTM backward pass (backpropagation
// through time).
//
// The trace page "Complete Trace: nn.LSTM" ("cuDNN Backward") computes the
// gradients of the input, of the initial states and of the weights from the
// gradients of (output, h_n, c_n) and the activations the forward saved; the
// pulsatrix "LSTMModule" reference walks the four gates and the cell carry
// backwards through time and accumulates every weight and bias gradient over
// all steps.  The derivatives are the chain rule of the cell equations on the
// warp-nn "Long Short-Term Memory (LSTM)" page:
//   h = o tanh(c),  c = f c_prev + i g
//   dc   = dc_next + dh o (1 - tanh^2 c)
//   dz_o = dh tanh(c) o (1 - o),  dz_i = dc g i (1 - i)
//   dz_g = dc i (1 - g^2),        dz_f = dc c_prev f (1 - f)
//   dc_prev = dc f,  dh_prev = W_hh^T dz,  dx = W_ih^T dz
//   dW_ih += dz x^T,  dW_hh += dz h_prev^T,  db_ih = db_hh += dz
//
//   k_bwd_cell  the first backward step of a scan, elementwise: dh, dc, dz
//   k_bwd_step  each backward step: the recurrent product dz_t W_hh of a
//               tile over the whole K on the matrix cores, then the cell
//               update of the step before it (or dh0 after the last)
//   k_transpose, k_hprev_t, k_cast_*  operand preparation for the weight
//               and input gradients, which are "NT" GEMMs on the projection
//               kernels (bf16 operands for bf16 parameters, else fp32)
//   k_colsum_part  the bias gradients, column sums of dz in fixed chunks
//   k_dropout_fwd, k_dropout_bwd  training dropout between layers: the trace
//               page's Performance Notes apply it to the input of every
//               layer above the first in training only; the draw is
//               Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
//               numbers: as easy as 1, 2, 3", SC 2011)
#include "device.h"
#include "kernels.h"

namespace lstm_amd {

// The cell part of backward step sb (sb = 0 is the last step of each
// direction's scan) at (d, b, j): from dh = dY + dh_rec (the recurrent
// product of the step after it) and the carried dc, the pre-activation
// gradients dz of the four gates and dc for the step before it.  It is split
// in two: CellIn holds what it reads besides the recurrent product.  None of
// that depends on the product, so a step kernel issues these loads before its
// product and they overlap its round trips.
struct CellIn {
    float dY, dhn, dhc, dcn, dc;         // dhn, dhc, dcn: 0 where the array is NULL
    float ig, fg, gg, og, c, c0, cpa;    // cpa: c of the scan's previous step (clamped time)
    int len;                             // 0 where lengths are NULL
};

// Every load is unconditional (any choice between them waits for the
// compiler's join of the paths, i.e. for the loads), and the choices are
// made in bwd_cell_store.  All of them are buffer loads with 32-bit offsets
// from wave-uniform bases (the step's time slices of acts and dY, the
// [D, B, H] arrays whole; the host keeps each within 2^31 bytes): 64-bit
// address arithmetic among the loads had the compiler pass a loaded register
// as a don't-care operand, i.e. wait for that load before the product's own
// loads went out.  sb and d must be uniform, b and j in range.
template <class G>
__device__ inline CellIn bwd_cell_load(const BwdCellArgs &a, int sb, int d, int b, int j) {
    const int T = a.T;
    const unsigned B = a.B, H = a.H, D = a.D;
    const int sf = T - 1 - sb;                   // the forward scan's step
    const int t = __builtin_amdgcn_readfirstlane(d == 0 ? sf : T - 1 - sf);  // its time index
    const int tp = d == 0 ? t - 1 : t + 1;       // time of the scan's previous step
    const int tpc = __builtin_amdgcn_readfirstlane(tp < 0 ? 0 : tp >= T ? T - 1 : tp);
    const unsigned ud = (unsigned)d, ub = (unsigned)b, uj = (unsigned)j;
    const unsigned sbytes = D * B * H * 4u, so = ((ud * B + ub) * H + uj) * 4u;  // [D, B, H]
    const unsigned arow = B * D * 5u * H;                                     // acts floats per step
    const unsigned ao = ((ub * D + ud) * 5u * H + uj) * 4u;
    const unsigned yrow = B * D * H;                                           // dY floats per step
    const unsigned yo = ((ub * D + ud) * H + uj) * 4u;
    const float *at = a.acts + (size_t)t * arow, *ap = a.acts + (size_t)tpc * arow;
    CellIn v;
    v.len = (int)__float_as_uint(load_f32_or0(a.len, B * 4u, ub * 4u));
    v.dhn = load_f32_or0(a.dhn, sbytes, so);
    v.dhc = load_f32_or0(a.dhc, sbytes, so);
    v.dcn = load_f32_or0(a.dcn, sbytes, so);
    v.dc = load_f32_or0(a.dc, sbytes, so);
    v.dY = load_f32_or0(a.dY + (size_t)t * yrow, yrow * 4u, yo);
    v.ig = load_f32_or0(at, arow * 4u, ao);
    v.fg = load_f32_or0(at, arow * 4u, ao + H * 4u);
    v.gg = load_f32_or0(at, arow * 4u, ao + 2u * H * 4u);
    v.og = load_f32_or0(at, arow * 4u, ao + 3u * H * 4u);
    v.c = load_f32_or0(at, arow * 4u, ao + 4u * H * 4u);
    v.c0 = load_f32_or0(a.c0, sbytes, so);
    v.cpa = load_f32_or0(ap, arow * 4u, ao + 4u * H * 4u);
    return v;
}

// The update itself, with v from bwd_cell_load (dz in the gradient dtype G).
template <class G>
__device__ inline void bwd_cell_store(const BwdCellArgs &a, int sb, int d, int b, int j, float dh_rec,
                                      const CellIn &v) {
    const int T = a.T, B = a.B, H = a.H, D = a.D;
    const int sf = T - 1 - sb;
    const int t = d == 0 ? sf : T - 1 - sf;
    const size_t dbj = ((size_t)d * B + b) * H + j;
    typename G::S *dz = static_cast<typename G::S *>(a.dz) + (((size_t)t * B + b) * D + d) * 4 * H + j;
    const float dcn = sb == 0 ? v.dcn : v.dc;  // the dc carried in (dc_n at the scan's last step)
    // With per-row lengths, a padded step (the forward left h and c alone
    // there and output 0) has zero dz; dc stays, and the gradient of h it
    // received goes on to the step before in a.dhc, joining that step's dh.
    if (a.len) {
        const float carried = sb == 0 ? v.dhn : v.dhc;
        if (t >= v.len) {
            if (sb == 0) a.dc[dbj] = dcn;
            a.dhc[dbj] = dh_rec + carried;
#pragma unroll
            for (int q = 0; q < 4; ++q) dz[(size_t)q * H] = G::from_f(0.f);
            return;
        }
        a.dhc[dbj] = 0.f;
        if (sb > 0) dh_rec += carried;  // at sb = 0, dh_n joins below
    }
    float dh = v.dY + dh_rec;
    if (sb == 0) dh += v.dhn;
    const float ig = v.ig, fg = v.fg, gg = v.gg, og = v.og;
    const float cprev = sf == 0 ? v.c0 : v.cpa;
    const float tc = tanh_f(v.c);
    const float dct = dcn + dh * og * (1.f - tc * tc);
    dz[0] = G::from_f(dct * gg * ig * (1.f - ig));
    dz[(size_t)H] = G::from_f(dct * cprev * fg * (1.f - fg));
    dz[(size_t)2 * H] = G::from_f(dct * ig * (1.f - gg * gg));
    dz[(size_t)3 * H] = G::from_f(dh * tc * og * (1.f - og));
    a.dc[dbj] = dct * fg;
}

template <class G>
__device__ inline void bwd_cell_update(const BwdCellArgs &a, int sb, int d, int b, int j, float dh_rec) {
    bwd_cell_store<G>(a, sb, d, b, j, dh_rec, bwd_cell_load<G>(a, sb, d, b, j));
}

// The first backward step of every (direction, batch row, unit): dh = dY + dh_n.
template <class G>
__global__ void k_bwd_cell(BwdCellArgs a) {
    const size_t n = (size_t)a.B * a.H;
    const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    if (i >= n) return;
    bwd_cell_update<G>(a, 0, (int)blockIdx.z, (int)(i / a.H), (int)(i % a.H), 0.f);
}

// Backward step sb: the recurrent product dh_prev = dz_t W_hh of step sb for
// one tile of 16 batch rows x 16 units of one direction, over the whole
// K = 4H (stacked gate order), then the cell update of step sb + 1 for the
// tile's cells -- or, after the scan's first step (sb = T - 1), dh0.
//   whT[d][j][k] = W_hh[d][k][j]: K-contiguous rows, as are dz's
// The BWD_WAVES waves take equal slices of K (16x16 MFMAs in the gradient
// dtype G, fp32 accumulation, fragments of 16-byte loads); their tiles meet
// in LDS, one output per thread of the first 256.  The cell update's own
// inputs are loaded before the product, so their round trip overlaps it.  A
// whole tile's K lives in one workgroup, so no partial sums leave it and
// nothing waits on another workgroup.  (Eight waves, two per SIMD, doubled
// the loads in flight and measured no faster: the fp32 product chain and the
// launch dominate a step.)
constexpr int BWD_WAVES = 4;

template <class G, class DT>
__global__ __launch_bounds__(BWD_WAVES * 64) void k_bwd_step(BwdMmArgs a, BwdCellArgs c, typename DT::S *dh0) {
    using S = typename G::S;
    constexpr int NW = BWD_WAVES;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int B = a.B, H = a.H, D = a.D, K = 4 * H;
    const int d = blockIdx.z;
    const int nmb = (B + 15) / 16, nub = (H + 15) / 16, ntile = nmb * nub;
    // with a K split, workgroups [0, ntile) own their tiles and finish them;
    // [ntile, 2 ntile) are their helpers (the same tile order, so a helper
    // runs on its owner's XCD when ntile is a multiple of 8)
    const int half = (int)blockIdx.x >= ntile ? 1 : 0;
    const int tile = (int)blockIdx.x - half * ntile;
    int mb, ub;
    {
        // the row blocks of one unit block run on the same XCD (round-robin
        // dispatch), so its W_hh^T rows are fetched into that XCD's L2 once
        const int bid = tile;
        if ((nub & 7) == 0) {
            const int idx = bid >> 3;
            ub = (bid & 7) + 8 * (idx / nmb);
            mb = idx % nmb;
        } else {
            ub = bid / nmb;
            mb = bid % nmb;
        }
    }
    const int b0 = mb * 16, u0 = ub * 16;
    const int b = b0 + (lane & 15);  // A row (batch row) of this lane
    const int j = u0 + (lane & 15);  // B row (unit) of this lane
    // this workgroup's K range (whole chunks), then each wave's
    const int kseg = (K + a.ksplit * G::KC - 1) / (a.ksplit * G::KC) * G::KC;
    const int kb = half * kseg, ke = min(K, kb + kseg);
    const int kq = (ke - kb + NW * G::KC - 1) / (NW * G::KC) * G::KC;
    const int k_lo = kb + w * kq, k_hi = min(ke, k_lo + kq);
    const int sf = a.T - 1 - a.sb;
    const int t = d == 0 ? sf : a.T - 1 - sf;
    constexpr unsigned es = sizeof(S);
    // dz rows (t, b, d) for b < B and whT rows (d, j) for j < H through buffer
    // resources: a row past B or H, or a chunk past the wave's K range, gets
    // an out-of-range offset and reads zeros without a memory access
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<S *>(static_cast<const S *>(a.dz) + ((size_t)t * B * D + d) * (size_t)K), (short)0,
        (int)(((size_t)(B - 1) * D * K + K) * es), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<S *>(static_cast<const S *>(a.whT) + (size_t)d * H * K), (short)0, (int)((size_t)H * K * es),
        0x00020000);
    const unsigned aoff = (unsigned)((size_t)b * D * K * es);
    const unsigned boff = (unsigned)((size_t)j * K * es);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // batches of 16 chunks: all 32 fragment loads are issued before the first
    // product of the batch; scheduling barriers keep the compiler from
    // interleaving them with the products into a chain of round trips
    constexpr int NBAT = 16;
    constexpr unsigned OOR = 0x7FFFFFF0u;
    auto issue = [&](int k0, u32x4 (&av)[NBAT], u32x4 (&bv)[NBAT]) {
#pragma unroll
        for (int q = 0; q < NBAT; ++q) {
            const int k = k0 + q * G::KC + (lane >> 4) * G::PER16;
            const bool kin = k < k_hi;
            av[q] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(kin && b < B ? aoff + es * k : OOR), 0, 0);
            bv[q] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(kin && j < H ? boff + es * k : OOR), 0, 0);
        }
    };
    auto multiply = [&](const u32x4 (&av)[NBAT], const u32x4 (&bv)[NBAT]) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < NBAT; ++q) acc = mma_chunk(G{}, acc, av[q], bv[q]);
        __builtin_amdgcn_sched_barrier(0);
    };
    // the cell update's own inputs (one cell per thread of the first 256)
    const int rb_ = (tid >> 4) & 15, ru = tid & 15;
    const int m = b0 + rb_, u = u0 + ru;
    const bool cell = tid < 256 && m < B && u < H && a.sb + 1 < a.T;
    const CellIn cin = bwd_cell_load<G>(c, min(a.sb + 1, a.T - 1), d, min(m, B - 1), min(u, H - 1));
    for (int k0 = k_lo; k0 < k_hi; k0 += NBAT * G::KC) {
        u32x4 av[NBAT], bv[NBAT];
        issue(k0, av, bv);
        multiply(av, bv);
    }
    // lane l, register v: batch row 4 (l / 16) + v, unit l % 16 of the tile
    __shared__ float red[NW][16][17];
#pragma unroll
    for (int v = 0; v < 4; ++v) red[w][4 * (lane >> 4) + v][lane & 15] = acc[v];
    __syncthreads();
    if (tid >= 256) return;
    float r = red[0][rb_][ru];  // the waves' K slices, added in order
#pragma unroll
    for (int q = 1; q < NW; ++q) r += red[q][rb_][ru];
    unsigned long long *pw = a.ksplit == 2 ? a.pbuf + ((size_t)d * ntile + tile) * 256 + tid : nullptr;
    const unsigned long long want = (unsigned long long)a.tag << 32;
    if (half) {  // helper: hand the partial sum over (every word, dead cells too)
        __hip_atomic_store(pw, want | __float_as_uint(r), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    if (m >= B || u >= H) return;
    if (a.ksplit == 2) {  // owner: the helper's half of K, added after this one's
        unsigned long long v = __hip_atomic_load(pw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((v & 0xFFFFFFFF00000000ull) != want) {
            const long long t0 = wall_clock64();
            do {
                __builtin_amdgcn_s_sleep(1);
                v = __hip_atomic_load(pw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((v & 0xFFFFFFFF00000000ull) == want) break;
                // an earlier wait gave up: the outputs are invalid, do not wait again
                if (wall_clock64() - t0 > a.timeout_ticks ||
                    (__hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 2u)) {
                    __hip_atomic_fetch_or(a.status, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            } while (true);
        }
        r += __uint_as_float((unsigned)v);
    }
    if (cell) bwd_cell_store<G>(c, a.sb + 1, d, m, u, r, cin);
    else if (dh0) dh0[((size_t)d * B + m) * H + u] = DT::from_f(r + (c.len ? c.dhc[((size_t)d * B + m) * H + u] : 0.f));
}

// out[c * ld_out + r] = in[r' * ld_in + c] for r < rows, c < cols (DI in, DO
// out), r' = r, or with bT > 0 the batch-first row of time-major row r =
// t*bB + b, i.e. b*bT + t
template <class DI, class DO>
__global__ void k_transpose(const typename DI::S *in, size_t ld_in, int rows, int cols, typename DO::S *out,
                            size_t ld_out, int bT, int bB) {
    __shared__ float tile[32][33];
    const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
    for (int rr = threadIdx.y; rr < 32; rr += 8) {
        const int r = r0 + rr, c = c0 + threadIdx.x;
        const size_t ri = bT > 0 ? (size_t)(r % bB) * bT + r / bB : (size_t)r;
        tile[rr][threadIdx.x] = (r < rows && c < cols) ? DI::to_f(in[ri * ld_in + c]) : 0.f;
    }
    __syncthreads();
    for (int cc = threadIdx.y; cc < 32; cc += 8) {
        const int c = c0 + cc, r = r0 + threadIdx.x;
        if (c < cols && r < rows) out[(size_t)c * ld_out + r] = DO::from_f(tile[threadIdx.x][cc]);
    }
}

// out[k][m] = h_prev of direction d for row m = t*B + b (k < H, m < T*B):
// the layer's output at the time of the scan's previous step, or h0 (NULL =
// zeros) at the scan's first step.
template <class DT, class DO>
__global__ void k_hprev_t(const typename DT::S *Y, size_t ldy, const typename DT::S *h0d, const int *len, int T,
                          int B, int H, int d, int bfirst, typename DO::S *out) {
    __shared__ float tile[32][33];
    const int m0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
    const int M = T * B;
    for (int mm = threadIdx.y; mm < 32; mm += 8) {
        const int m = m0 + mm, k = k0 + threadIdx.x;
        float v = 0.f;
        if (m < M && k < H) {
            const int t = m / B, b = m % B;
            const int tp = d == 0 ? t - 1 : t + 1;
            if (tp >= 0 && tp < T && !(len && tp >= len[b]))  // a padded predecessor kept h0
                v = DT::to_f(Y[trow(tp, b, T, B, bfirst != 0) * ldy + (size_t)d * H + k]);
            else if (h0d) v = DT::to_f(h0d[(size_t)b * H + k]);
        }
        tile[mm][threadIdx.x] = v;
    }
    __syncthreads();
    for (int kk = threadIdx.y; kk < 32; kk += 8) {
        const int k = k0 + kk, m = m0 + threadIdx.x;
        if (k < H && m < M) out[(size_t)k * M + m] = DO::from_f(tile[threadIdx.x][kk]);
    }
}

// Column sums in fixed row chunks: part[c][col] = sum over rows r in chunk c
// (rows c*chunk .. ) of a[r * ld + col], each summed in row order; the
// chunks are then added in order by k_ksum (deterministic).
template <class DT>
__global__ void k_colsum_part(const typename DT::S *a, size_t ld, int rows, int cols, int chunk, float *part) {
    const int col = blockIdx.x * blockDim.x + threadIdx.x;
    if (col >= cols) return;
    const int r0 = blockIdx.y * chunk, r1 = min(rows, r0 + chunk);
    float s = 0.f;
    int r = r0;
    for (; r + 8 <= r1; r += 8) {  // eight loads in flight, added in row order
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = DT::to_f(a[(size_t)(r + q) * ld + col]);
#pragma unroll
        for (int q = 0; q < 8; ++q) s += v[q];
    }
    for (; r < r1; ++r) s += DT::to_f(a[(size_t)r * ld + col]);
    part[(size_t)blockIdx.y * cols + col] = s;
}

template <class DT>
__global__ void k_cast_to(const float *in, typename DT::S *out, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        out[i] = DT::from_f(in[i]);
}

template <class DT>
__global__ void k_cast_from(const typename DT::S *in, float *out, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        out[i] = DT::to_f(in[i]);
}

// Sum of K-split slabs in a fixed order (deterministic), rounded once to the
// output dtype.
template <class DT>
__global__ void k_ksum(const float *part, int ns, size_t slab, size_t n, typename DT::S *out) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        float v = part[i];
        int sp = 1;
        for (; sp + 8 <= ns; sp += 8) {  // eight loads in flight, added in slab order
            float w[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) w[q] = part[(size_t)(sp + q) * slab + i];
#pragma unroll
            for (int q = 0; q < 8; ++q) v += w[q];
        }
        for (; sp < ns; ++sp) v += part[(size_t)sp * slab + i];
        out[i] = DT::from_f(v);
    }
}

// Philox4x64-10 block: ten rounds, each two 64 x 64 -> 128-bit products of
// counter words 0 and 2 by the published multipliers, mixed with the other
// two words and the key; the key advances by the published Weyl constants
// after every round.
__device__ inline void philox4x64_10(unsigned long long (&c)[4], unsigned long long k0, unsigned long long k1) {
    constexpr unsigned long long M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const unsigned long long hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
        const unsigned long long hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
        const unsigned long long n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
        k0 += 0x9E3779B97F4A7C15ull;
        k1 += 0xBB67AE8584CAA73Bull;
    }
}

// Training dropout of layer `layer`'s output y (n elements, flat index e over
// [T][B][D*H]): the block with counter (e / 4, layer, call, 0) and key
// (seed, 0) gives four words; word e % 4 keeps e when (word >> 11) >= thr,
// i.e. (word >> 11) * 2^-53 >= p with thr = ceil(p * 2^53), an exact integer
// form of the comparison.  xd = kept ? y * scale : 0 (the next layer's
// input), keep = the decision (read again by the backward pass).
template <class DT>
__global__ void k_dropout_fwd(const typename DT::S *y, typename DT::S *xd, unsigned char *keep, size_t n,
                              unsigned long long seed, unsigned long long call, int layer, unsigned long long thr,
                              float scale, int T, int B, int width, int bfirst) {
    const size_t nblk = (n + 3) / 4;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < nblk; i += (size_t)gridDim.x * blockDim.x) {
        unsigned long long c[4] = {(unsigned long long)i, (unsigned long long)layer, call, 0ull};
        philox4x64_10(c, seed, 0ull);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const size_t e = 4 * i + q;
            if (e >= n) break;
            const bool kept = (c[q] >> 11) >= thr;
            // e counts time-major ([T][B][width]); y and xd may be batch-first
            size_t ye = e;
            if (bfirst) {
                const size_t r = e / width;
                ye = trow((int)(r / B), (int)(r % B), T, B, true) * width + e % width;
            }
            xd[ye] = DT::from_f(kept ? DT::to_f(y[ye]) * scale : 0.f);
            keep[e] = kept ? 1 : 0;
        }
    }
}

// The gradient reaching layer `layer`'s output through the dropout.
__global__ void k_dropout_bwd(float *g, const unsigned char *keep, size_t n, float scale) {
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x)
        g[e] = keep[e] ? g[e] * scale : 0.f;
}

// ---------------------------------------------------------------- launchers
static unsigned grid1(size_t n, unsigned cap = 8192) {
    const size_t g = (n + 255) / 256;
    return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

hipError_t launch_bwd_cell(const BwdCellArgs &a, int gdt, hipStream_t s) {
    const size_t n = (size_t)a.B * a.H;
    const dim3 grid((unsigned)((n + 255) / 256), 1, a.D);
    if (gdt == DT_BF16) hipLaunchKernelGGL(k_bwd_cell<BF16>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_bwd_cell<F32>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bwd_step(const BwdMmArgs &a, const BwdCellArgs &c, void *dh0, int gdt, int dtype, hipStream_t s) {
    if (c.dz != a.dz || c.T != a.T || c.B != a.B || c.H != a.H || c.D != a.D) return hipErrorInvalidValue;
    if (gdt == DT_BF16 && a.H % 2 != 0) return hipErrorInvalidValue;  // whole bf16 fragments over K = 4H
    if (a.ksplit != 1 && (a.ksplit != 2 || !a.pbuf || !a.status || a.tag == 0)) return hipErrorInvalidValue;
    dim3 grid(((a.B + 15) / 16) * ((a.H + 15) / 16) * a.ksplit, 1, a.D);
    if (gdt == DT_BF16 && dtype == DT_BF16)
        hipLaunchKernelGGL((k_bwd_step<BF16, BF16>), grid, dim3(BWD_WAVES * 64), 0, s, a, c, static_cast<uint16_t *>(dh0));
    else if (gdt == DT_BF16)
        return hipErrorInvalidValue;
    else if (dtype == DT_BF16)
        hipLaunchKernelGGL((k_bwd_step<F32, BF16>), grid, dim3(BWD_WAVES * 64), 0, s, a, c, static_cast<uint16_t *>(dh0));
    else
        hipLaunchKernelGGL((k_bwd_step<F32, F32>), grid, dim3(BWD_WAVES * 64), 0, s, a, c, static_cast<float *>(dh0));
    return hipGetLastError();
}

hipError_t launch_transpose(const void *in, size_t ld_in, int rows, int cols, void *out, size_t ld_out, int in_dtype,
                            int out_dtype, hipStream_t s, int bT, int bB) {
    dim3 grid((cols + 31) / 32, (rows + 31) / 32), block(32, 8);
    if (grid.y > 65535u || (bT > 0 && (long long)bT * bB != rows)) return hipErrorInvalidValue;
    const bool bi = in_dtype == DT_BF16, bo = out_dtype == DT_BF16;
    if (bi && bo)
        hipLaunchKernelGGL((k_transpose<BF16, BF16>), grid, block, 0, s, static_cast<const uint16_t *>(in), ld_in, rows,
                           cols, static_cast<uint16_t *>(out), ld_out, bT, bB);
    else if (bi)
        hipLaunchKernelGGL((k_transpose<BF16, F32>), grid, block, 0, s, static_cast<const uint16_t *>(in), ld_in, rows,
                           cols, static_cast<float *>(out), ld_out, bT, bB);
    else if (bo)
        hipLaunchKernelGGL((k_transpose<F32, BF16>), grid, block, 0, s, static_cast<const float *>(in), ld_in, rows,
                           cols, static_cast<uint16_t *>(out), ld_out, bT, bB);
    else
        hipLaunchKernelGGL((k_transpose<F32, F32>), grid, block, 0, s, static_cast<const float *>(in), ld_in, rows,
                           cols, static_cast<float *>(out), ld_out, bT, bB);
    return hipGetLastError();
}

// Rows of width elements between the time-major [T][B] and batch-first
// [B][T] orders (to_tm: batch-first in, time-major out), with a dtype change.
template <class DI, class DO>
__global__ void k_permute_rows(const typename DI::S *in, typename DO::S *out, int T, int B, int width, int to_tm) {
    const size_t n = (size_t)T * B * width;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const size_t r = e / width, k = e % width;
        const int t = (int)(r / B), b = (int)(r % B);  // time-major row r = t*B + b
        const size_t rb = (size_t)b * T + t;
        if (to_tm) out[e] = DO::from_f(DI::to_f(in[rb * width + k]));
        else out[rb * width + k] = DO::from_f(DI::to_f(in[e]));
    }
}

hipError_t launch_permute_rows(const void *in, void *out, int T, int B, int width, int in_dtype, int out_dtype,
                               bool to_time_major, hipStream_t s) {
    const size_t n = (size_t)T * B * width;
    if (n == 0) return hipSuccess;
    const unsigned g = (unsigned)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
    const int tm = to_time_major ? 1 : 0;
    const bool bi = in_dtype == DT_BF16, bo = out_dtype == DT_BF16;
    if (bi && !bo)
        hipLaunchKernelGGL((k_permute_rows<BF16, F32>), dim3(g), dim3(256), 0, s, static_cast<const uint16_t *>(in),
                           static_cast<float *>(out), T, B, width, tm);
    else if (!bi && bo)
        hipLaunchKernelGGL((k_permute_rows<F32, BF16>), dim3(g), dim3(256), 0, s, static_cast<const float *>(in),
                           static_cast<uint16_t *>(out), T, B, width, tm);
    else if (!bi && !bo)
        hipLaunchKernelGGL((k_permute_rows<F32, F32>), dim3(g), dim3(256), 0, s, static_cast<const float *>(in),
                           static_cast<float *>(out), T, B, width, tm);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_hprev_t(const void *Y, size_t ldy, const void *h0d, const int *len, int T, int B, int H, int d,
                          void *out, int dtype, int out_dtype, hipStream_t s, bool batch_first) {
    const int bf = batch_first ? 1 : 0;
    dim3 grid(((size_t)T * B + 31) / 32, (H + 31) / 32), block(32, 8);
    if (grid.y > 65535u) return hipErrorInvalidValue;
    if (dtype == DT_BF16 && out_dtype == DT_BF16)
        hipLaunchKernelGGL((k_hprev_t<BF16, BF16>), grid, block, 0, s, static_cast<const uint16_t *>(Y), ldy,
                           static_cast<const uint16_t *>(h0d), len, T, B, H, d, bf, static_cast<uint16_t *>(out));
    else if (dtype == DT_BF16)
        hipLaunchKernelGGL((k_hprev_t<BF16, F32>), grid, block, 0, s, static_cast<const uint16_t *>(Y), ldy,
                           static_cast<const uint16_t *>(h0d), len, T, B, H, d, bf, static_cast<float *>(out));
    else if (out_dtype == DT_F32)
        hipLaunchKernelGGL((k_hprev_t<F32, F32>), grid, block, 0, s, static_cast<const float *>(Y), ldy,
                           static_cast<const float *>(h0d), len, T, B, H, d, bf, static_cast<float *>(out));
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_colsum_part(const void *a, size_t ld, int rows, int cols, int nchunks, float *part, int dtype,
                              hipStream_t s) {
    if (rows < 1 || cols < 1 || nchunks < 1) return hipErrorInvalidValue;
    const int chunk = (rows + nchunks - 1) / nchunks;
    dim3 grid((cols + 255) / 256, (unsigned)((rows + chunk - 1) / chunk));
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(k_colsum_part<BF16>, grid, dim3(256), 0, s, static_cast<const uint16_t *>(a), ld, rows,
                           cols, chunk, part);
    else
        hipLaunchKernelGGL(k_colsum_part<F32>, grid, dim3(256), 0, s, static_cast<const float *>(a), ld, rows, cols,
                           chunk, part);
    return hipGetLastError();
}

hipError_t launch_cast_to(const float *in, void *out, size_t n, int dtype, hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(k_cast_to<BF16>, dim3(grid1(n)), dim3(256), 0, s, in, static_cast<uint16_t *>(out), n);
    else
        hipLaunchKernelGGL(k_cast_to<F32>, dim3(grid1(n)), dim3(256), 0, s, in, static_cast<float *>(out), n);
    return hipGetLastError();
}

hipError_t launch_ksum(const float *part, int ns, size_t slab, size_t n, void *out, int dtype, hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (ns < 1 || (ns > 1 && slab < n)) return hipErrorInvalidValue;
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(k_ksum<BF16>, dim3(grid1(n)), dim3(256), 0, s, part, ns, slab, n,
                           static_cast<uint16_t *>(out));
    else
        hipLaunchKernelGGL(k_ksum<F32>, dim3(grid1(n)), dim3(256), 0, s, part, ns, slab, n, static_cast<float *>(out));
    return hipGetLastError();
}

hipError_t launch_dropout_fwd(const void *y, void *xd, unsigned char *keep, int T, int B, int width,
                              unsigned long long seed, unsigned long long call, int layer, unsigned long long thr,
                              float scale, int dtype, bool batch_first, hipStream_t s) {
    const size_t n = (size_t)T * B * width;
    if (n == 0) return hipSuccess;
    const unsigned g = grid1((n + 3) / 4);
    const int bf = batch_first ? 1 : 0;
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(k_dropout_fwd<BF16>, dim3(g), dim3(256), 0, s, static_cast<const uint16_t *>(y),
                           static_cast<uint16_t *>(xd), keep, n, seed, call, layer, thr, scale, T, B, width, bf);
    else
        hipLaunchKernelGGL(k_dropout_fwd<F32>, dim3(g), dim3(256), 0, s, static_cast<const float *>(y),
                           static_cast<float *>(xd), keep, n, seed, call, layer, thr, scale, T, B, width, bf);
    return hipGetLastError();
}

hipError_t launch_dropout_bwd(float *g, const unsigned char *keep, size_t n, float scale, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_dropout_bwd, dim3(grid1(n)), dim3(256), 0, s, g, keep, n, scale);
    return hipGetLastError();
}

hipError_t launch_cast_from(const void *in, float *out, size_t n, int dtype, hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(k_cast_from<BF16>, dim3(grid1(n)), dim3(256), 0, s, static_cast<const uint16_t *>(in),
                           out, n);
    else
        hipLaunchKernelGGL(k_cast_from<F32>, dim3(grid1(n)), dim3(256), 0, s, static_cast<const float *>(in), out,
                           n);
    return hipGetLastError();
}

}  // namespace lstm_amd
