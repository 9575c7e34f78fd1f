// kernels.hip -- gfx950 kernels of the LSTM forward pass.
//
//   k_proj  the input projection of one layer for every time step at once:
//           G = X W_ih^T + b_ih + b_hh, an "NT" GEMM on the matrix cores.
//           The gate pre-activation splits into a part that depends only on
//           x_t and a part that depends on h_{t-1} (warp-nn "Long Short-Term
//           Memory (LSTM)", equation block); the first part carries no
//           recurrence and is hoisted out of the time loop.  The MXNet blog
//           "LSTM Forward Computation" ("Basic Operators") concatenates the
//           four gate matrices into one so that one product serves all gates;
//           the warp-nn parameter table fixes the [i; f; g; o] row blocks.
//   k_rec   the recurrence of one layer: per step S = h_{t-1} W_hh^T on the
//           matrix cores, then the gate nonlinearities and the cell update
//           (same equation block) fused into the epilogue; the reverse
//           direction runs in the same launch on its own workgroups.  Either
//           one launch per step, or one persistent launch per layer with the
//           W_hh slices resident in LDS; workgroups hand h_t to each other
//           through step-tagged words instead of a grid barrier.
//   k_rec_step  one step of the recurrence as a GEMM with the cell update
//           fused, for layers whose W_hh does not stay on chip.
//   k_fill  clears the status word and the exchange buffer.
//   k_mask_padded  zeroes the outputs of padded steps (variable-length rows).
#include "device.h"
#include "kernels.h"
#include "rec.h"

namespace lstm_amd {

// Split of one projection workgroup: direction, K range and output slab.
struct ProjSplit {
    int d, kb, kc;  // direction, first K index, K length of this split
    size_t goff;    // float offset of this split's output slab
};
__device__ inline ProjSplit proj_split(const ProjArgs &a) {
    if (a.kchunk <= 0) return ProjSplit{(int)blockIdx.z, 0, a.K, 0};
    const int ns = (a.K + a.kchunk - 1) / a.kchunk, z = blockIdx.z, sp = z % ns;
    return ProjSplit{z / ns, sp * a.kchunk, min(a.K - sp * a.kchunk, a.kchunk), (size_t)sp * a.M * a.D * a.N};
}

// ===========================================================================
// Projection GEMM.  128x128 output tile per 256-thread workgroup; each of the
// four waves owns a 64x64 quadrant as 4x4 MFMA tiles of 16x16.  A stage holds
// 128 bytes of K per row (two chunks), double-buffered in LDS; 16-byte
// segments are XOR-swizzled by row so that the fragment reads of 16 rows at
// one K offset spread over the banks.
// ===========================================================================
template <class DT, bool VEC>
__global__ __launch_bounds__(256) void k_proj(ProjArgs a) {
    using S = typename DT::S;
    constexpr int BM = 128, BN = 128, SEG = 8;
    constexpr int KS = SEG * DT::PER16;
    __shared__ u32x4 sA[2][BM * SEG];
    __shared__ u32x4 sB[2][BN * SEG];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const ProjSplit sp = proj_split(a);
    const int d = sp.d;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int M = a.M, N = a.N, K = sp.kc, ldw = a.K;
    const S *X = static_cast<const S *>(a.X) + sp.kb;
    const S *W = static_cast<const S *>(a.W[d]) + sp.kb;
    float *const Gs = a.G + sp.goff;

    u32x4 ra[4], rb[4];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int seg = tid + 256 * i, row = seg >> 3, sg = seg & 7;
            const int k = k0 + sg * DT::PER16;
            ra[i] = (m0 + row < M) ? load_frag<DT>(X + (size_t)(m0 + row) * a.ldx, k, K, VEC) : zero;
            rb[i] = (n0 + row < N) ? load_frag<DT>(W + (size_t)(n0 + row) * ldw, k, K, VEC) : zero;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int seg = tid + 256 * i, row = seg >> 3, sg = seg & 7;
            const int pos = row * SEG + (sg ^ ((row >> 1) & 7));
            sA[buf][pos] = ra[i];
            sB[buf][pos] = rb[i];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + KS - 1) / KS;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * KS);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            u32x4 af[4], bw[4];
            const int sg = 4 * c + (lane >> 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm * 64 + 16 * i + (lane & 15);
                af[i] = sA[buf][row * SEG + (sg ^ ((row >> 1) & 7))];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wn * 64 + 16 * j + (lane & 15);
                bw[j] = sB[buf][row * SEG + (sg ^ ((row >> 1) & 7))];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mma_chunk(DT{}, acc[i][j], af[i], bw[j]);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: lane l holds rows 4*(l/16)+v, column l%16 of each 16x16 tile.
    const S *bi = static_cast<const S *>(a.b_ih[d]);
    const S *bh = static_cast<const S *>(a.b_hh[d]);
    float bias[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + 16 * j + (lane & 15);
        bias[j] = (bi && n < N) ? DT::to_f(bi[n]) + (bh ? DT::to_f(bh[n]) : 0.f) : 0.f;
    }
    const size_t ldg = (size_t)a.D * N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn * 64 + 16 * j + (lane & 15);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + wm * 64 + 16 * i + 4 * (lane >> 4) + v;
                if (m < M && n < N) Gs[(size_t)m * ldg + (size_t)d * N + n] = acc[i][j][v] + bias[j];
            }
        }
}

// Output-tile order of the 256x256 GEMM kernels.  Workgroups are dispatched
// round-robin over the 8 XCDs, each with its own L2.  The 32 workgroups an
// XCD runs together get a 4x8 block of tiles (4 row bands x 8 column bands),
// so the 4 A panels and 8 W panels they stream are fetched into that L2 once
// and shared, instead of every tile of one row band streaming all of W.
__device__ inline void gemm_tile_order(int bid, int ntm, int ntn, int &tm, int &tn) {
    const int ntiles = ntm * ntn;
    if (ntm % 4 == 0 && ntn % 8 == 0 && ntiles % 256 == 0) {
        const int xcd = bid & 7, li = bid >> 3;
        const int grp = (li >> 5) * 8 + xcd, pos = li & 31;
        const int ngc = ntn / 8;
        tm = (grp / ngc) * 4 + (pos >> 3);
        tn = (grp % ngc) * 8 + (pos & 7);
    } else {
        int tile = bid;
        if ((ntiles & 7) == 0) tile = (tile & 7) * (ntiles >> 3) + (tile >> 3);
        tm = tile / ntn;
        tn = tile % ntn;
    }
}

// ===========================================================================
// Projection GEMM, large tiles.  256x256 output tile per 256-thread workgroup;
// each wave owns a 128x128 quadrant as 4x4 tiles of 32x32 (v_mfma_f32_32x32x16
// _bf16 / v_mfma_f32_32x32x2_f32), which halves the LDS and L2 bytes per FLOP
// of the 128x128 kernel.  Stages of 128 bytes of K per row are double-buffered
// in LDS (128 KiB), with 16-byte segments XOR-swizzled by (row/2) % 8 so that a
// wave's fragment read of 16 consecutive rows touches 16 distinct bank groups.
// Tiles are ordered by gemm_tile_order: 4x8 tile blocks per XCD.
// ===========================================================================
template <class DT, bool VEC>
__global__ __launch_bounds__(256) void k_proj_big(ProjArgs a) {
    using S = typename DT::S;
    constexpr int BM = 256, BN = 256, SEG = 8;
    constexpr int KS = SEG * DT::PER16;
    extern __shared__ __align__(16) unsigned char smem[];
    u32x4 *lds = reinterpret_cast<u32x4 *>(smem);
    constexpr int STAGE = (BM + BN) * SEG;  // 16-byte segments per stage

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const ProjSplit sp = proj_split(a);
    const int d = sp.d;
    const int M = a.M, N = a.N, K = sp.kc, ldw = a.K;
    int tm, tn;
    gemm_tile_order(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const S *X = static_cast<const S *>(a.X) + sp.kb;
    const S *W = static_cast<const S *>(a.W[d]) + sp.kb;
    float *const Gs = a.G + sp.goff;

    u32x4 ra[8], rb[8];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int seg = tid + 256 * i, row = seg >> 3, sg = seg & 7;
            const int k = k0 + sg * DT::PER16;
            ra[i] = (m0 + row < M) ? load_frag<DT>(X + (size_t)(m0 + row) * a.ldx, k, K, VEC) : zero;
            rb[i] = (n0 + row < N) ? load_frag<DT>(W + (size_t)(n0 + row) * ldw, k, K, VEC) : zero;
        }
    };
    auto swz = [](int row, int sg) { return row * SEG + (sg ^ ((row >> 1) & 7)); };
    auto sstore = [&](int buf) {
        u32x4 *sa = lds + buf * STAGE, *sb = sa + BM * SEG;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int seg = tid + 256 * i, row = seg >> 3, sg = seg & 7;
            sa[swz(row, sg)] = ra[i];
            sb[swz(row, sg)] = rb[i];
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = (K + KS - 1) / KS;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * KS);
        const u32x4 *sa = lds + buf * STAGE, *sb = sa + BM * SEG;
#pragma unroll
        for (int c = 0; c < 4; ++c) {  // 32 bytes of K per row per sub-chunk
            u32x4 af[4], bw[4];
            const int sg = 2 * c + (lane >> 5);
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = sa[swz(wm * 128 + 32 * i + (lane & 31), sg)];
#pragma unroll
            for (int j = 0; j < 4; ++j) bw[j] = sb[swz(wn * 128 + 32 * j + (lane & 31), sg)];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mma32_chunk(DT{}, acc[i][j], af[i], bw[j]);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    const S *bi = static_cast<const S *>(a.b_ih[d]);
    const S *bh = static_cast<const S *>(a.b_hh[d]);
    const size_t ldg = (size_t)a.D * N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 128 + 32 * j + (lane & 31);
        const float bias = (bi && n < N) ? DT::to_f(bi[n]) + (bh ? DT::to_f(bh[n]) : 0.f) : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm * 128 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m < M && n < N) Gs[(size_t)m * ldg + (size_t)d * N + n] = acc[i][j][v] + bias;
            }
    }
}

// ===========================================================================
// Projection GEMM, large tiles fed by direct-to-LDS loads.  Same 256x256 tile,
// wave split and MFMA work as k_proj_big, but global data goes straight into
// LDS (buffer_load_dwordx4 ... lds): stage k+1 streams into the other LDS
// buffer while stage k is multiplied, with no register staging and one
// barrier per stage.  A load instruction fills 1 KiB of LDS (64 lanes x 16
// bytes, consecutive), i.e. 8 rows of a stage; each lane fetches the global
// segment whose swizzled home is its slot.  Rows past M or N and K past K
// read as zeros (offsets beyond the buffer resource).  Needs K and the row
// strides to be multiples of 16 bytes.
// ===========================================================================
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr unsigned OOR_STEP = 0x80000000u;  // a buffer offset past any resource: reads zero

template <class DT>
__global__ __launch_bounds__(256) void k_proj_dma(ProjArgs a) {
    using S = typename DT::S;
    constexpr int BM = 256, BN = 256, SEG = 8;
    constexpr int KS = SEG * DT::PER16;
    constexpr int STAGE = (BM + BN) * SEG;  // 16-byte segments per stage
    constexpr unsigned OOR = 0x80000000u;   // past any resource: reads zero
    extern __shared__ __align__(16) unsigned char smem[];
    u32x4 *lds = reinterpret_cast<u32x4 *>(smem);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const ProjSplit sp = proj_split(a);
    const int d = sp.d;
    const int M = a.M, N = a.N, K = sp.kc, ldw = a.K;
    int tm, tn;
    gemm_tile_order(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int es = (int)sizeof(S);
    const S *X = static_cast<const S *>(a.X) + (size_t)m0 * a.ldx + sp.kb;
    const S *W = static_cast<const S *>(a.W[d]) + (size_t)n0 * ldw + sp.kb;
    float *const Gs = a.G + sp.goff;
    // bytes from this split's first element to the end of its last row's K range
    const unsigned xbytes = (unsigned)(((size_t)(min(BM, M - m0) - 1) * a.ldx + K) * es);
    const unsigned wbytes = (unsigned)(((size_t)(min(BN, N - n0) - 1) * ldw + K) * es);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<S *>(X), (short)0, (int)xbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<S *>(W), (short)0, (int)wbytes, 0x00020000);

    // this lane's slot in each 1 KiB block: row (lane / 8) of the block, swizzled segment (lane % 8)
    const int brow = lane >> 3, pseg = lane & 7;
    auto issue = [&](int kt, int buf) {
        u32x4 *sa = lds + buf * STAGE, *sb = sa + BM * SEG;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int blk = w + 4 * i;  // 32 blocks of 8 rows per operand
            const int row = blk * 8 + brow;
            const int lseg = pseg ^ ((row >> 1) & 7);
            const int k = kt * KS + lseg * DT::PER16;
            const unsigned ox = k < K ? (unsigned)(((size_t)row * a.ldx + k) * es) : OOR;
            const unsigned ow = k < K ? (unsigned)(((size_t)row * ldw + k) * es) : OOR;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t *)(sa + blk * 64), 16, ox, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t *)(sb + blk * 64), 16, ow, 0, 0, 0);
        }
    };
    auto swz = [](int row, int sg) { return row * SEG + (sg ^ ((row >> 1) & 7)); };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = (K + KS - 1) / KS;
    issue(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of stage kt are in LDS
        __syncthreads();                 // everyone's are, and stage kt-1 is no longer read
        if (kt + 1 < nk) issue(kt + 1, buf ^ 1);
        const u32x4 *sa = lds + buf * STAGE, *sb = sa + BM * SEG;
        // fragments of sub-chunk c+1 are read while sub-chunk c is multiplied
        u32x4 af[2][4], bw[2][4];
        auto frags = [&](int c, u32x4 (&fa)[4], u32x4 (&fb)[4]) {
            const int sg = 2 * c + (lane >> 5);
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = sa[swz(wm * 128 + 32 * i + (lane & 31), sg)];
#pragma unroll
            for (int j = 0; j < 4; ++j) fb[j] = sb[swz(wn * 128 + 32 * j + (lane & 31), sg)];
        };
        frags(0, af[0], bw[0]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (c + 1 < 4) frags(c + 1, af[(c + 1) & 1], bw[(c + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);  // keep the read-ahead in front of the products
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mma32_chunk(DT{}, acc[i][j], af[c & 1][i], bw[c & 1][j]);
        }
    }

    const S *bi = static_cast<const S *>(a.b_ih[d]);
    const S *bh = static_cast<const S *>(a.b_hh[d]);
    const size_t ldg = (size_t)a.D * N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 128 + 32 * j + (lane & 31);
        const float bias = (bi && n < N) ? DT::to_f(bi[n]) + (bh ? DT::to_f(bh[n]) : 0.f) : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm * 128 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m < M && n < N) Gs[(size_t)m * ldg + (size_t)d * N + n] = acc[i][j][v] + bias;
            }
    }
}

// ===========================================================================
// Projection GEMM, k_proj_dma with the next stage's loads spread over the
// products.  With one wave per SIMD, the issue of a stage's 16 direct-to-LDS
// loads (and their address arithmetic) in one burst leaves the matrix pipe
// idle for that time.  Here each lane's load offsets are computed once, a
// stage is addressed by advancing the buffer resources' base, and the next
// stage's loads go out in four groups, each behind the four products of one
// row tile of the stage's first K sub-chunk, where they issue while those
// products run.  Same tile, LDS layout, operand order and sums as k_proj_dma
// (its results, bit for bit).  A stage that reaches past K (a ragged last
// stage) is issued with per-segment checks, as in k_proj_dma.
// ===========================================================================
template <class DT>
__global__ __launch_bounds__(256) void k_proj_il(ProjArgs a) {
    using S = typename DT::S;
    constexpr int BM = 256, BN = 256, SEG = 8;
    constexpr int KS = SEG * DT::PER16;
    constexpr int STAGE = (BM + BN) * SEG;  // 16-byte segments per stage
    constexpr unsigned OOR = 0x80000000u;   // past any resource: reads zero
    extern __shared__ __align__(16) unsigned char smem[];
    u32x4 *lds = reinterpret_cast<u32x4 *>(smem);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const ProjSplit sp = proj_split(a);
    const int d = sp.d;
    const int M = a.M, N = a.N, K = sp.kc, ldw = a.K;
    int tm, tn;
    gemm_tile_order(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int es = (int)sizeof(S);
    const S *X = static_cast<const S *>(a.X) + (size_t)m0 * a.ldx + sp.kb;
    const S *W = static_cast<const S *>(a.W[d]) + (size_t)n0 * ldw + sp.kb;
    float *const Gs = a.G + sp.goff;
    const unsigned xbytes = (unsigned)(((size_t)(min(BM, M - m0) - 1) * a.ldx + K) * es);
    const unsigned wbytes = (unsigned)(((size_t)(min(BN, N - n0) - 1) * ldw + K) * es);

    // this lane's slot in each 1 KiB block: row (lane / 8) of the block, swizzled segment (lane % 8)
    const int brow = lane >> 3, pseg = lane & 7;
    unsigned vx[8], vw[8];  // byte offsets of this lane's 8 segments of a stage (stage 0)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (w + 4 * i) * 8 + brow;
        const int lseg = pseg ^ ((row >> 1) & 7);
        vx[i] = (unsigned)(((size_t)row * a.ldx + lseg * DT::PER16) * es);
        vw[i] = (unsigned)(((size_t)row * ldw + lseg * DT::PER16) * es);
    }
    // every segment of stage kt lies inside K: the resources start at K offset
    // kt * KS (rows past M or N stay past the shortened resources: ldx, ldw >= K)
    auto issue_part = [&](int kt, int buf, int part) {
        u32x4 *sa = lds + buf * STAGE, *sb = sa + BM * SEG;
        const unsigned kb = (unsigned)(kt * KS * es);
        const __amdgpu_buffer_rsrc_t rx =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<S *>(X + (size_t)kt * KS), (short)0, (int)(xbytes - kb), 0x00020000);
        const __amdgpu_buffer_rsrc_t rw =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<S *>(W + (size_t)kt * KS), (short)0, (int)(wbytes - kb), 0x00020000);
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int i = 2 * part + ii, blk = w + 4 * i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t *)(sa + blk * 64), 16, vx[i], 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t *)(sb + blk * 64), 16, vw[i], 0, 0, 0);
        }
    };
    // a stage reaching past K: each segment checked
    const __amdgpu_buffer_rsrc_t rx0 = __builtin_amdgcn_make_buffer_rsrc(const_cast<S *>(X), (short)0, (int)xbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw0 = __builtin_amdgcn_make_buffer_rsrc(const_cast<S *>(W), (short)0, (int)wbytes, 0x00020000);
    auto issue_checked = [&](int kt, int buf) {
        u32x4 *sa = lds + buf * STAGE, *sb = sa + BM * SEG;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int blk = w + 4 * i;
            const int row = blk * 8 + brow;
            const int lseg = pseg ^ ((row >> 1) & 7);
            const int k = kt * KS + lseg * DT::PER16;
            const unsigned ox = k < K ? (unsigned)(((size_t)row * a.ldx + k) * es) : OOR;
            const unsigned ow = k < K ? (unsigned)(((size_t)row * ldw + k) * es) : OOR;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx0, (lds_void_t *)(sa + blk * 64), 16, ox, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw0, (lds_void_t *)(sb + blk * 64), 16, ow, 0, 0, 0);
        }
    };
    auto swz = [](int row, int sg) { return row * SEG + (sg ^ ((row >> 1) & 7)); };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = (K + KS - 1) / KS;
    const int nfull = K / KS;  // stages entirely inside K
    if (nfull > 0) {
#pragma unroll
        for (int part = 0; part < 4; ++part) issue_part(0, 0, part);
    } else {
        issue_checked(0, 0);
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of stage kt are in LDS
        __syncthreads();                 // everyone's are, and stage kt-1 is no longer read
        const bool nxt = kt + 1 < nk, nxt_full = kt + 1 < nfull;
        if (nxt && !nxt_full) issue_checked(kt + 1, buf ^ 1);
        const u32x4 *sa = lds + buf * STAGE, *sb = sa + BM * SEG;
        u32x4 af[2][4], bw[2][4];
        auto frags = [&](int c, u32x4 (&fa)[4], u32x4 (&fb)[4]) {
            const int sg = 2 * c + (lane >> 5);
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = sa[swz(wm * 128 + 32 * i + (lane & 31), sg)];
#pragma unroll
            for (int j = 0; j < 4; ++j) fb[j] = sb[swz(wn * 128 + 32 * j + (lane & 31), sg)];
        };
        frags(0, af[0], bw[0]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (c + 1 < 4) frags(c + 1, af[(c + 1) & 1], bw[(c + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);  // keep the read-ahead in front of the products
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mma32_chunk(DT{}, acc[i][j], af[c & 1][i], bw[c & 1][j]);
                if (c == 0) {
                    // a quarter of the next stage's loads behind each row tile's products
                    if (nxt_full) issue_part(kt + 1, buf ^ 1, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }

    const S *bi = static_cast<const S *>(a.b_ih[d]);
    const S *bh = static_cast<const S *>(a.b_hh[d]);
    const size_t ldg = (size_t)a.D * N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 128 + 32 * j + (lane & 31);
        const float bias = (bi && n < N) ? DT::to_f(bi[n]) + (bh ? DT::to_f(bh[n]) : 0.f) : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm * 128 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m < M && n < N) Gs[(size_t)m * ldg + (size_t)d * N + n] = acc[i][j][v] + bias;
            }
    }
}

// ===========================================================================
// Recurrence, one step as a GEMM.  For layers whose W_hh does not stay on
// chip, each step is one launch of this kernel: S = h_{t-1} W_hh^T for a block
// of BM = 32*WM batch rows and 32 hidden units, followed in the same kernel by
// the gate nonlinearities and the cell update (the equation block of the
// warp-nn LSTM page) for those cells.  h_{t-1} is read from y of the previous
// step (or h0), which the launch boundary has made visible, so no exchange
// words are needed.  The block's 128 rows of W_hh are gathered gate-major
// (row r: gate r / 32, unit u0 + r % 32), so that in the 32x32 MFMA output
// layout each lane holds all four gate pre-activations of its cells and the
// cell update needs no data exchange.  Operands stream from global memory
// straight into LDS (128 bytes of K per row per stage, XOR-swizzled 16-byte
// segments as in k_proj_dma) through a ring of NST stages, so that several
// stages of loads are in flight while one is multiplied.  The four waves are
// WM row slices x (4/WM) K slices; K slices' partial sums meet in LDS.  The
// per-step traffic is bounded by the L2-to-CU bandwidth, (BM + 128) rows of
// K per workgroup: taller blocks read less in total, shorter ones spread the
// products over more CUs.  c is carried across launches in cstate.
//
// The other recurrent modes of the trace page's RNNBase (MODE 1 GRU, 2
// RNN_TANH, 3 RNN_RELU) run through the same kernel with NG = 3 or 1 gate
// blocks (BR = 32 NG rows of W_hh per block) and their own update: G holds
// x W_ih^T + b_ih only, and b_hh is added here, because the GRU's candidate
// multiplies its hidden contribution, bias included, by the reset gate.
// Their state is h alone, read back from y of the previous step.
// ===========================================================================
template <class DT, int WM, int MODE>
__global__ __launch_bounds__(256) void k_rec_step(RecArgs a) {
    using S = typename DT::S;
    constexpr int NG = MODE == 0 ? 4 : MODE == 1 ? 3 : 1;  // gate blocks
    constexpr int WKS = 4 / WM;                  // K slices
    constexpr int BM = 32 * WM, BR = 32 * NG, SEG = 8;  // A rows, W rows per block; segments per row
    constexpr int KS = SEG * DT::PER16;          // K per stage
    constexpr int STAGE = (BM + BR) * SEG;       // 16-byte segments per stage
    constexpr int NST = WM == 4 ? 4 : 5;         // stages in the LDS ring
    constexpr int LPS = (BM + BR) / 32;          // 1 KiB loads per wave per stage
    extern __shared__ __align__(16) unsigned char smem[];
    u32x4 *lds = reinterpret_cast<u32x4 *>(smem);

    // the wave index in a scalar register: the operand choice below depends on it
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w % WM, wk = w / WM;
    const int H = a.H, B = a.B, T = a.T, D = a.D;
    const int d = blockIdx.z;
    const int s = a.s_begin;
    const int t = d == 0 ? s : T - 1 - s;
    const int nmb = (B + BM - 1) / BM, nub = (H + 31) / 32;
    int mb, ub;
    {
        const int bid = blockIdx.x;
        if ((nub & 7) == 0) {
            // the row blocks of one unit block run on the same XCD (round-robin
            // dispatch), so its W_hh rows are fetched into that XCD's L2 once
            const int idx = bid >> 3;
            ub = (bid & 7) + 8 * (idx / nmb);
            mb = idx % nmb;
        } else {
            ub = bid / nmb;
            mb = bid % nmb;
        }
    }
    const int b0 = mb * BM, u0 = ub * 32;
    const int es = (int)sizeof(S);
    const size_t ldy = (size_t)D * H;

    f32x16 acc[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;

    // h_{t-1}: rows b0.. of y at the previous step, or of h0 at s = 0
    const S *hsrc = nullptr;
    size_t lda = 0;
    if (s > 0) {
        const int tp = d == 0 ? s - 1 : T - s;
        hsrc = static_cast<const S *>(a.Y) + trow(tp, b0, T, B, a.bfirst) * ldy + (size_t)d * H;
        lda = a.bfirst ? (size_t)T * ldy : ldy;
    } else if (a.h0) {
        hsrc = static_cast<const S *>(a.h0) + ((size_t)d * B + b0) * H;
        lda = H;
    }

    // G of the cells this lane finishes (below): independent of the product,
    // so they are loaded while it runs (streamed once: non-temporal).  Cells
    // past B or H read a clamped valid address; their values go unused.
    constexpr int VPW = 16 / WKS;  // result registers finished per wave
    const size_t ldg = (size_t)D * NG * H;
    // bytes of h_{t-1} this block may read (its rows of y or h0)
    const unsigned hbytes = hsrc ? (unsigned)((((size_t)min(BM, B - b0) - 1) * lda + H) * sizeof(S)) : 0u;
    // The LSTM's carried c (c0 at the first step, NULL: zeros) likewise, and
    // for the other modes b_hh and the cell's h_{t-1} (NULL: zeros).
    float gv[VPW][NG], cpv[VPW], hpv[VPW], bhv[NG];
    auto load_gv = [&]() {
        const int uc = min(u0 + (lane & 31), H - 1);
        const float *cb = s == 0 ? a.c0 : a.cstate;
#pragma unroll
        for (int vv = 0; vv < VPW; ++vv) {
            const int v = VPW * wk + vv;
            const int mc = min(b0 + wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), B - 1);
            const float *g = a.G + trow(t, mc, T, B, a.bfirst) * ldg + (size_t)d * NG * H + uc;
#pragma unroll
            for (int j = 0; j < NG; ++j) gv[vv][j] = __builtin_nontemporal_load(g + (size_t)j * H);
            if constexpr (MODE == 0)
                cpv[vv] = load_f32_or0(cb, (unsigned)((size_t)D * B * H * 4),
                                       (unsigned)((((size_t)d * B + mc) * H + uc) * 4));
            else
                hpv[vv] = load_s_or0<DT>(hsrc, hbytes, (unsigned)(((size_t)(mc - b0) * lda + uc) * sizeof(S)));
        }
        if constexpr (MODE != 0)
#pragma unroll
            for (int j = 0; j < NG; ++j)
                bhv[j] = load_s_or0<DT>(a.b_hh[d], (unsigned)((size_t)NG * H * sizeof(S)),
                                        (unsigned)(((size_t)j * H + uc) * sizeof(S)));
    };

    if (hsrc) {
        const int rows = min(BM, B - b0);
        const unsigned abytes = (unsigned)((((size_t)rows - 1) * lda + H) * es);
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<S *>(hsrc), (short)0, (int)abytes, 0x00020000);
        const S *W = static_cast<const S *>(a.whh[d]);
        const unsigned wbytes = (unsigned)((size_t)NG * H * H * es);
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<S *>(W), (short)0, (int)wbytes, 0x00020000);

        // this lane's slot in each 1 KiB block: row (lane / 8) of the block, swizzled segment (lane % 8)
        const int brow = lane >> 3, pseg = lane & 7;
        auto issue = [&](int kt, int buf) {
            u32x4 *st = lds + buf * STAGE;
#pragma unroll
            for (int i = 0; i < LPS; ++i) {
                const int blk = w + 4 * i;  // BM/8 blocks of A rows, then 16 of W rows
                const int row = blk * 8 + brow;
                const int lseg = pseg ^ ((row >> 1) & 7);
                const int k = kt * KS + lseg * DT::PER16;
                unsigned off;
                if (blk < BM / 8) {
                    off = k < H ? (unsigned)(((size_t)row * lda + k) * es) : OOR_STEP;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t *)(st + blk * 64), 16, off, 0, 0, 0);
                } else {
                    const int r = row - BM, u = u0 + (r & 31);
                    off = (k < H && u < H) ? (unsigned)(((size_t)((r >> 5) * H + u) * H + k) * es) : OOR_STEP;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t *)(st + blk * 64), 16, off, 0, 0, 0);
                }
            }
        };
        auto swz = [](int row, int sg) { return row * SEG + (sg ^ ((row >> 1) & 7)); };

        const int nk = (H + KS - 1) / KS;
#pragma unroll
        for (int k = 0; k < NST - 1; ++k)
            if (k < nk) issue(k, k);
        // after the first stages (a wait the compiler may place among these
        // loads then covers loads the first products need anyway); the stage
        // waits below stay conservative: the extra loads only make the first
        // stages wait for them as well
        load_gv();
        for (int kt = 0; kt < nk; ++kt) {
            const int buf = kt % NST;
            // this wave's loads of stage kt are in LDS once at most the loads of
            // the later stages already issued (up to NST-2 of them) are pending
            constexpr int VM = LPS * (NST - 2);
            static_assert(VM < 64, "vmcnt field");
            if (kt + NST - 2 < nk) __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
            else __builtin_amdgcn_s_waitcnt(0);
            // Everyone's are, and stage kt-1 is no longer read (its fragments were
            // consumed by the products of the previous iteration).  A bare barrier:
            // the workgroup fence of __syncthreads would also wait for the loads
            // of the later stages, which must stay in flight.  The signal fences
            // keep the compiler from moving LDS accesses across it.
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (kt + NST - 1 < nk) issue(kt + NST - 1, (kt + NST - 1) % NST);
            const u32x4 *sa = lds + buf * STAGE, *sb = sa + BM * SEG;
            // this wave's 32-byte sub-chunks of the stage: wk, wk + WKS, ...
            constexpr int NC = 4 / WKS;
            u32x4 af[NC], bw[NC][NG];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int sg = 2 * (wk + WKS * c) + (lane >> 5);
                af[c] = sa[swz(wm * 32 + (lane & 31), sg)];
#pragma unroll
                for (int j = 0; j < NG; ++j) bw[c][j] = sb[swz(32 * j + (lane & 31), sg)];
            }
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int j = 0; j < NG; ++j) acc[j] = mma32_chunk(DT{}, acc[j], af[c], bw[c][j]);
        }
        __syncthreads();  // the stage buffers are reused below
    }

    if (!hsrc) load_gv();  // no product at this step

    // With two K slices, wave (wm, wk) finishes the result registers
    // v in [8 wk, 8 wk + 8) and hands the other half to its partner.
    float *red = reinterpret_cast<float *>(smem);  // [4 waves][32 values][64 lanes]
    const int partner = wm + WM * (1 - wk);
    if (WKS == 2) {
#pragma unroll
        for (int j = 0; j < NG; ++j)
#pragma unroll
            for (int vv = 0; vv < 8; ++vv) red[((size_t)w * 32 + j * 8 + vv) * 64 + lane] = acc[j][8 * (1 - wk) + vv];
        __syncthreads();
    }
    const int u = u0 + (lane & 31);
    const bool last = s == T - 1;
#pragma unroll
    for (int vv = 0; vv < VPW; ++vv) {
        const int v = VPW * wk + vv;
        const int m = b0 + wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m >= B || u >= H) continue;
        float pre[NG];
#pragma unroll
        for (int j = 0; j < NG; ++j)
            pre[j] = acc[j][v] + (WKS == 2 ? red[((size_t)partner * 32 + j * 8 + vv) * 64 + lane] : 0.f);
        const float *g = gv[vv];  // G of gate block j at g[j]
        const size_t si = ((size_t)d * B + m) * H + u;
        if constexpr (MODE != 0) {
            // hidden contributions with b_hh; h_{t-1} of this cell for the GRU
#pragma unroll
            for (int j = 0; j < NG; ++j) pre[j] += bhv[j];
            const S hprev = DT::from_f(hpv[vv]);  // exact: an S value widened
            float hv;
            if constexpr (MODE == 1) {
                const float rg = sigmoid_f(g[0] + pre[0]);
                const float zg = sigmoid_f(g[1] + pre[1]);
                const float ng = tanh_f(g[2] + rg * pre[2]);
                hv = (1.f - zg) * ng + zg * hpv[vv];
            } else if constexpr (MODE == 2) {
                hv = tanh_f(g[0] + pre[0]);
            } else {
                hv = fmaxf(g[0] + pre[0], 0.f);
            }
            // a padded step of this row keeps h, which y carries to the next
            // step (padded outputs are zeroed after the last layer)
            const S hs = (a.len && t >= a.len[m]) ? hprev : DT::from_f(hv);
            static_cast<S *>(a.Y)[trow(t, m, T, B, a.bfirst) * ldy + (size_t)d * H + u] = hs;
            if (last && a.hn) static_cast<S *>(a.hn)[si] = hs;
        } else {
            const float cp = cpv[vv];
            const float ig = sigmoid_f(pre[0] + g[0]);
            const float fg = sigmoid_f(pre[1] + g[1]);
            const float gg = tanh_f(pre[2] + g[2]);
            const float og = sigmoid_f(pre[3] + g[3]);
            float cn = fg * cp + ig * gg;
            S hs = DT::from_f(og * tanh_f(cn));
            if (a.len && t >= a.len[m]) {
                // padded step of this row: the state stays; y carries the unchanged
                // h because the next step reads h_{t-1} from y (padded outputs are
                // zeroed after the last layer)
                cn = cp;
                hs = hsrc ? hsrc[(size_t)(m - b0) * lda + u] : (S)0;
            }
            a.cstate[si] = cn;
            if (a.acts) {  // training: the activations the backward pass needs
                float *ap = a.acts + (((size_t)t * B + m) * D + d) * 5 * H + u;
                ap[0] = ig;
                ap[(size_t)H] = fg;
                ap[(size_t)2 * H] = gg;
                ap[(size_t)3 * H] = og;
                ap[(size_t)4 * H] = cn;
            }
            static_cast<S *>(a.Y)[trow(t, m, T, B, a.bfirst) * ldy + (size_t)d * H + u] = hs;
            if (last) {
                if (a.hn) static_cast<S *>(a.hn)[si] = hs;
                if (a.cn) a.cn[si] = cn;
            }
        }
    }
}

// y[t][b][:] = 0 for t >= len[b]; one 16-bit unit per thread (rows of bf16
// or fp32 values are whole units)
__global__ void k_mask_padded(uint16_t *y, const int *len, int T, int B, size_t row_units, int batch_first) {
    const size_t n = (size_t)T * B * row_units;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const size_t row = i / row_units;
        const int t = batch_first ? (int)(row % T) : (int)(row / B);
        const int b = batch_first ? (int)(row / T) : (int)(row % B);
        if (t >= len[b]) y[i] = 0;
    }
}

__global__ void k_fill(unsigned *p, size_t n, unsigned v) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// ===========================================================================
// Projection GEMM, 256x256 tiles fed through a ring of NST direct-to-LDS
// stages.  The double buffer of k_proj_dma drains every load before each
// stage's barrier, so each wave keeps at most one stage of loads in flight
// and the next stage must land within one stage of products.  Here a stage
// holds 64 bytes of K per row (32 KiB for both operands), NST - 1 stages are
// issued ahead, and the wait before a stage's barrier lets the later stages'
// loads stay pending (a vmcnt bound instead of a full drain).
// Each 1 KiB load fills 16 rows of 4 segments; segment s of row r sits at
// r * 4 + (s ^ ((r / 4) % 4)), so 16 consecutive rows reading one segment
// touch 16 distinct 16-byte bank groups.  The products and the epilogue are
// those of k_proj_dma.  With BN = 128 (each wave a 128x64 quadrant) and three
// stages a workgroup takes 72 KiB of LDS, so two share a CU and one's waits
// overlap the other's products.
// ===========================================================================
template <class DT, int NST, int BN>
__global__ __launch_bounds__(256, BN == 128 ? 2 : 1) void k_proj_ring(ProjArgs a) {
    using S = typename DT::S;
    constexpr int BM = 256, SEG = 4;
    constexpr int NJ = BN / 64;                  // 32-column tiles per wave
    constexpr int KS = SEG * DT::PER16;
    constexpr int STAGE = (BM + BN) * SEG;       // 16-byte segments per stage
    constexpr int LPS = (BM + BN) / 16 / 4;      // 1 KiB loads per wave per stage
    static_assert((BM + BN) % 64 == 0, "whole loads per wave");
    constexpr unsigned OOR = 0x80000000u;        // past any resource: reads zero
    extern __shared__ __align__(16) unsigned char smem[];
    u32x4 *lds = reinterpret_cast<u32x4 *>(smem);

    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 1, wn = w & 1;
    const ProjSplit sp = proj_split(a);
    const int d = sp.d;
    const int M = a.M, N = a.N, K = sp.kc, ldw = a.K;
    int tm, tn;
    gemm_tile_order(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int es = (int)sizeof(S);
    const S *X = static_cast<const S *>(a.X) + (size_t)m0 * a.ldx + sp.kb;
    const S *W = static_cast<const S *>(a.W[d]) + (size_t)n0 * ldw + sp.kb;
    float *const Gs = a.G + sp.goff;
    const unsigned xbytes = (unsigned)(((size_t)(min(BM, M - m0) - 1) * a.ldx + K) * es);
    const unsigned wbytes = (unsigned)(((size_t)(min(BN, N - n0) - 1) * ldw + K) * es);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<S *>(X), (short)0, (int)xbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<S *>(W), (short)0, (int)wbytes, 0x00020000);

    // this lane's slot in each 1 KiB block: row (lane / 4) of the block, swizzled segment (lane % 4)
    const int brow = lane >> 2, pseg = lane & 3;
    auto issue = [&](int kt, int buf) {
        u32x4 *st = lds + buf * STAGE;
#pragma unroll
        for (int i = 0; i < LPS; ++i) {
            const int blk = w + 4 * i;  // BM/16 blocks of 16 X rows, then BN/16 of W rows
            const bool isx = blk < BM / 16;
            const int row = (isx ? blk : blk - BM / 16) * 16 + brow;
            const int lseg = pseg ^ ((row >> 2) & 3);
            const int k = kt * KS + lseg * DT::PER16;
            const unsigned off = k < K ? (unsigned)(((size_t)row * (isx ? a.ldx : ldw) + k) * es) : OOR;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isx ? rx : rw, (lds_void_t *)(st + blk * 64), 16, off, 0, 0, 0);
        }
    };
    auto swz = [](int row, int sg) { return row * SEG + (sg ^ ((row >> 2) & 3)); };

    f32x16 acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = (K + KS - 1) / KS;
#pragma unroll
    for (int k = 0; k < NST - 1; ++k)
        if (k < nk) issue(k, k);
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt % NST;
        // this wave's loads of stage kt are in LDS once at most the loads of
        // the later stages already issued (up to NST-2 of them) are pending
        constexpr int VM = LPS * (NST - 2);
        static_assert(VM < 64, "vmcnt field");
        if (kt + NST - 2 < nk) __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
        else __builtin_amdgcn_s_waitcnt(0);
        // everyone's are, and stage kt-1 is no longer read; a bare barrier, so
        // that the later stages' loads stay in flight
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (kt + NST - 1 < nk) issue(kt + NST - 1, (kt + NST - 1) % NST);
        const u32x4 *sa = lds + buf * STAGE, *sb = sa + BM * SEG;
        u32x4 af[2][4], bw[2][NJ];
        auto frags = [&](int c, u32x4 (&fa)[4], u32x4 (&fb)[NJ]) {
            const int sg = 2 * c + (lane >> 5);
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = sa[swz(wm * 128 + 32 * i + (lane & 31), sg)];
#pragma unroll
            for (int j = 0; j < NJ; ++j) fb[j] = sb[swz(wn * (BN / 2) + 32 * j + (lane & 31), sg)];
        };
        frags(0, af[0], bw[0]);
        frags(1, af[1], bw[1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) acc[i][j] = mma32_chunk(DT{}, acc[i][j], af[c][i], bw[c][j]);
    }

    const S *bi = static_cast<const S *>(a.b_ih[d]);
    const S *bh = static_cast<const S *>(a.b_hh[d]);
    const size_t ldg = (size_t)a.D * N;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int n = n0 + wn * (BN / 2) + 32 * j + (lane & 31);
        const float bias = (bi && n < N) ? DT::to_f(bi[n]) + (bh ? DT::to_f(bh[n]) : 0.f) : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm * 128 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (m < M && n < N) Gs[(size_t)m * ldg + (size_t)d * N + n] = acc[i][j][v] + bias;
            }
    }
}

// ===========================================================================
// Host-side launch helpers.
// ===========================================================================
static int proj_nsplit(const ProjArgs &a) { return a.kchunk > 0 ? (a.K + a.kchunk - 1) / a.kchunk : 1; }

template <class DT, int NST, int BN>
static hipError_t launch_proj_ring(const ProjArgs &a, hipStream_t s) {
    const void *fn = reinterpret_cast<const void *>(&k_proj_ring<DT, NST, BN>);
    const size_t smem = (size_t)NST * (256 + BN) * 4 * 16;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    dim3 grid(((a.M + 255) / 256) * ((a.N + BN - 1) / BN), 1, a.D * proj_nsplit(a));
    hipLaunchKernelGGL((k_proj_ring<DT, NST, BN>), grid, dim3(256), smem, s, a);
    return hipGetLastError();
}

template <class DT, bool VEC>
static hipError_t launch_proj_t(const ProjArgs &a, bool big, bool dma, int ring, hipStream_t s) {
    const int zd = a.D * proj_nsplit(a);
    if (big && dma && VEC && ring == 4) return launch_proj_ring<DT, 4, 256>(a, s);
    if (big && dma && VEC && ring == 5) return launch_proj_ring<DT, 5, 256>(a, s);
    if (big && dma && VEC && ring == 6) return launch_proj_ring<DT, 3, 128>(a, s);
    if (big && dma && VEC && (ring == 7 || ring == 0)) {
        const void *fn = reinterpret_cast<const void *>(&k_proj_il<DT>);
        const size_t smem = 2 * (256 + 256) * 8 * 16;
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        dim3 grid(((a.M + 255) / 256) * ((a.N + 255) / 256), 1, zd);
        hipLaunchKernelGGL((k_proj_il<DT>), grid, dim3(256), smem, s, a);
        return hipGetLastError();
    }
    if (big && dma && VEC) {
        const void *fn = reinterpret_cast<const void *>(&k_proj_dma<DT>);
        const size_t smem = 2 * (256 + 256) * 8 * 16;
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        dim3 grid(((a.M + 255) / 256) * ((a.N + 255) / 256), 1, zd);
        hipLaunchKernelGGL((k_proj_dma<DT>), grid, dim3(256), smem, s, a);
    } else if (big) {
        const void *fn = reinterpret_cast<const void *>(&k_proj_big<DT, VEC>);
        const size_t smem = 2 * (256 + 256) * 8 * 16;
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        dim3 grid(((a.M + 255) / 256) * ((a.N + 255) / 256), 1, zd);
        hipLaunchKernelGGL((k_proj_big<DT, VEC>), grid, dim3(256), smem, s, a);
    } else {
        dim3 grid((a.N + 127) / 128, (a.M + 127) / 128, zd);
        hipLaunchKernelGGL((k_proj<DT, VEC>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

// 256x256 tiles once they give every CU at least one tile (or on request);
// their direct-to-LDS form needs 16-byte rows and the byte offsets of one
// tile within 31 bits.
static void proj_choose(int M, int N, int K, int ldx, int D, int dtype, int variant, bool vec, bool *big,
                        bool *dma) {
    const long long big_tiles = (long long)((M + 255) / 256) * ((N + 255) / 256) * D;
    *big = variant >= 2 || (variant == 0 && big_tiles >= 256);
    const size_t es = dtype == DT_BF16 ? 2 : 4;
    *dma = *big && vec && variant != 2 && (size_t)256 * ldx * es < (1u << 31) && (size_t)256 * K * es < (1u << 31);
}

// the direct-to-LDS variants: 4 / 5 stages of 256x256 tiles, 6: three
// stages of 256x128 tiles, 7 (and automatic, 0): k_proj_il, the double
// buffer with its loads interleaved with the products; 3: k_proj_dma, the
// double buffer with each stage's loads issued together
static int proj_ring(int variant) { return variant >= 4 && variant <= 7 ? variant : 0; }

int proj_kchunk(int M, int N, int K) {
    const long long tiles = (long long)((M + 255) / 256) * ((N + 255) / 256);
    if (tiles >= 128 || K < 512) return 0;
    long long ns = 256 / tiles;
    if (ns > K / 256) ns = K / 256;
    if (ns < 2) return 0;
    const int kc = (int)(((K + ns - 1) / ns + 63) / 64 * 64);
    return kc < K ? kc : 0;
}

const char *proj_kernel_name(int M, int N, int K, int D, int dtype, int variant) {
    const int per16 = dtype == DT_BF16 ? 8 : 4;
    bool big, dma;
    proj_choose(M, N, K, K, D, dtype, variant, K % per16 == 0, &big, &dma);
    return dma ? (variant == 7 || variant == 0 ? "k_proj_il" : proj_ring(variant) ? "k_proj_ring" : "k_proj_dma")
               : big ? "k_proj_big" : "k_proj";
}

hipError_t launch_proj(const ProjArgs &a, int dtype, int variant, hipStream_t s) {
    const int per16 = dtype == DT_BF16 ? 8 : 4;
    bool vec = (a.K % per16 == 0) && (a.ldx % per16 == 0) && ((uintptr_t)a.X % 16 == 0);
    for (int d = 0; d < a.D; ++d) vec = vec && ((uintptr_t)a.W[d] % 16 == 0);
    if (a.kchunk < 0 || a.kchunk % 64 != 0 || (a.kchunk > 0 && (a.b_ih[0] || a.b_ih[1])))
        return hipErrorInvalidValue;
    bool big, dma;
    proj_choose(a.M, a.N, a.K, a.ldx, a.D * proj_nsplit(a), dtype, variant, vec, &big, &dma);
    const int ring = proj_ring(variant);
    if (dtype == DT_BF16)
        return vec ? launch_proj_t<BF16, true>(a, big, dma, ring, s) : launch_proj_t<BF16, false>(a, big, dma, ring, s);
    return vec ? launch_proj_t<F32, true>(a, big, dma, ring, s) : launch_proj_t<F32, false>(a, big, dma, ring, s);
}

int rec_rows_per_wg(RecTile t) { return 16 * (4 / t.WK) * t.MTW; }

// Chunks fetched per batch by one wave: all of a K-split wave's chunks when
// they fit in registers, two for the tall batch tiles.
int rec_chunk_batch(RecTile t) { return t.MTW >= 4 ? 2 : 8; }

RecGeom rec_geom(RecTile t, int H, int dtype, bool want_two_partial_buffers) {
    RecGeom g{};
    const int kc = dtype == DT_BF16 ? 32 : 16;
    g.kch = (H + kc - 1) / kc;
    const int cb = rec_chunk_batch(t);
    const int cpw = (g.kch + t.WK - 1) / t.WK;
    g.nbatch = (cpw + cb - 1) / cb;
    g.kchp = t.WK * g.nbatch * cb;
    // W_hh in registers when a wave's chunks are one batch of at most 32
    // fragments (128 VGPRs)
    g.wreg = g.nbatch == 1 && cb * t.NT <= 32 ? 1 : 0;
    const size_t wbytes = g.wreg ? 0 : (size_t)g.kchp * t.NT * 1024;
    const size_t pbytes = (size_t)t.WK * rec_rows_per_wg(t) * (16 * t.NT + 4) * 4;
    g.part_bufs = (want_two_partial_buffers && wbytes + 2 * pbytes <= kRecLdsLimit) ? 2 : 1;
    g.smem = wbytes + g.part_bufs * pbytes;
    return g;
}

bool rec_tile_supported(RecTile t) {
#define LSTM_T_OK(wk, mtw, nt) if (t.WK == wk && t.MTW == mtw && t.NT == nt) return true;
    LSTM_REC_TILES(LSTM_T_OK)
#undef LSTM_T_OK
    return false;
}

int rec_fused_chunks(RecTile t) {
#define LSTM_F_OK(wk, mtw, nt) if (t.WK == wk && t.MTW == mtw && t.NT == nt) return LSTM_FX_OF(nt);
    LSTM_REC_FUSED_TILES(LSTM_F_OK)
#undef LSTM_F_OK
    return 0;
}

// wide: the wide bf16 exchange words (no effect for fp32, whose words carry any value)
static const void *rec_kernel(RecTile t, int dtype, bool wreg, bool fused, bool wide) {
    if (dtype == DT_BF16) return wide ? rec_kernel_bf16_wide(t, wreg, fused) : rec_kernel_bf16(t, wreg, fused);
    return rec_kernel_f32(t, wreg, fused);
}

hipError_t rec_max_coresident(RecTile t, size_t smem, int dtype, bool wreg, bool fused, bool wide,
                              int *blocks_per_cu) {
    const void *fn = rec_kernel(t, dtype, wreg, fused, wide);
    if (!fn) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, 256, smem);
}

hipError_t launch_rec(const RecArgs &a, RecTile t, size_t smem, int dtype, bool cooperative, hipStream_t s) {
    const void *fn = rec_kernel(t, dtype, a.wreg != 0, a.ncx > 0, a.xwide != 0);
    if (!fn) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    dim3 grid(a.NGB * a.D * a.P), block(256);
    RecArgs copy = a;
    void *args[] = {&copy};
    if (cooperative) return hipLaunchCooperativeKernel(fn, grid, block, args, (unsigned)smem, s);
    return hipLaunchKernel(fn, grid, block, args, smem, s);
}

bool rec_step_gemm_ok(const RecArgs &a, int dtype) {
    const size_t es = dtype == DT_BF16 ? 2 : 4;
    // the A rows of one block (y of the previous step) must be addressable by
    // one buffer resource: 127 row strides, T rows apart when batch_first
    const size_t astride = (size_t)a.D * a.H * (a.bfirst ? (size_t)a.T : 1);
    const size_t ng = a.mode == 0 ? 4 : a.mode == 1 ? 3 : 1;
    bool ok = ((size_t)a.H * es) % 16 == 0 && ng * a.H * a.H * es < (1u << 31) &&
              ((size_t)128 * astride * es) < (1u << 31) && (size_t)a.D * a.B * a.H * 4 < (1u << 31) &&
              (uintptr_t)a.Y % 16 == 0 &&
              (!a.h0 || (uintptr_t)a.h0 % 16 == 0);
    for (int d = 0; d < a.D; ++d) ok = ok && (uintptr_t)a.whh[d] % 16 == 0;
    return ok;
}

// 64-row blocks on all CUs: measured faster than 128-row blocks (which read
// less in total) at B = 256 -- each CU's load rate is the limit.
int rec_step_rows(int) { return 64; }

template <class DT, int WM, int MODE>
static hipError_t launch_step_t(const RecArgs &a, hipStream_t s) {
    const void *fn = reinterpret_cast<const void *>(&k_rec_step<DT, WM, MODE>);
    constexpr int NG = MODE == 0 ? 4 : MODE == 1 ? 3 : 1;
    // the stage ring, and at least the K-slice exchange of the epilogue
    const size_t ring = (size_t)(WM == 4 ? 4 : 5) * (32 * WM + 32 * NG) * 8 * 16;
    const size_t red = WM == 2 ? (size_t)4 * 32 * 64 * sizeof(float) : 0;
    const size_t smem = ring > red ? ring : red;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    const int bm = 32 * WM;
    dim3 grid(((a.B + bm - 1) / bm) * ((a.H + 31) / 32), 1, a.D), block(256);
    RecArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(fn, grid, block, args, smem, s);
}

template <class DT>
static hipError_t launch_step_mode(const RecArgs &a, hipStream_t s) {
    switch (a.mode) {
        case 0: return launch_step_t<DT, 2, 0>(a, s);
        case 1: return launch_step_t<DT, 2, 1>(a, s);
        case 2: return launch_step_t<DT, 2, 2>(a, s);
        case 3: return launch_step_t<DT, 2, 3>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rec_step_gemm(const RecArgs &a, int dtype, hipStream_t s) {
    if (dtype == DT_BF16) return launch_step_mode<BF16>(a, s);
    return launch_step_mode<F32>(a, s);
}

hipError_t launch_mask_padded(void *y, const int *len, int T, int B, size_t row_bytes, bool batch_first,
                              hipStream_t s) {
    if (row_bytes % 2 != 0) return hipErrorInvalidValue;
    const size_t n = (size_t)T * B * (row_bytes / 2);
    const unsigned blocks = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(k_mask_padded, dim3(blocks), dim3(256), 0, s, static_cast<uint16_t *>(y), len, T, B,
                       row_bytes / 2, batch_first ? 1 : 0);
    return hipGetLastError();
}

// Parameter copies padded with zero rows (the GRU and the plain RNNs run on
// the LSTM's four gate slots): job blockIdx.y copies its first valid*cols
// elements and zeroes the rest of rows*cols.
constexpr int kPadJobs = 32;
struct PadBatch {
    PadJob j[kPadJobs];
};
template <class DT>
__global__ void k_pad_rows(PadBatch a) {
    using S = typename DT::S;
    const PadJob jb = a.j[blockIdx.y];
    const S *src = static_cast<const S *>(jb.src);
    S *dst = static_cast<S *>(jb.dst);
    const size_t n = (size_t)jb.rows * jb.cols, nv = (size_t)jb.valid * jb.cols;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x)
        dst[e] = e < nv ? src[e] : (S)0;
}

hipError_t launch_pad_rows(const PadJob *jobs, int n, int dtype, hipStream_t s) {
    for (int j0 = 0; j0 < n; j0 += kPadJobs) {
        PadBatch b{};
        const int m = n - j0 < kPadJobs ? n - j0 : kPadJobs;
        size_t most = 0;
        for (int k = 0; k < m; ++k) {
            b.j[k] = jobs[j0 + k];
            if (b.j[k].valid < 0 || b.j[k].valid > b.j[k].rows) return hipErrorInvalidValue;
            const size_t e = (size_t)b.j[k].rows * b.j[k].cols;
            most = e > most ? e : most;
        }
        const unsigned gx = (unsigned)((most + 255) / 256 < 1024 ? (most + 255) / 256 : 1024);
        dim3 grid(gx < 1 ? 1 : gx, (unsigned)m);
        if (dtype == DT_BF16) hipLaunchKernelGGL(k_pad_rows<BF16>, grid, dim3(256), 0, s, b);
        else hipLaunchKernelGGL(k_pad_rows<F32>, grid, dim3(256), 0, s, b);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_fill_u32(unsigned *p, size_t n, unsigned v, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024);
    hipLaunchKernelGGL(k_fill, dim3(blocks), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

}  // namespace lstm_amd
