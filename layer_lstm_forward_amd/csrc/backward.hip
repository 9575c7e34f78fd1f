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
//   k_bwd_cell  one backward step, elementwise: dh, dc, dz for every cell
//   k_bwd_mm    the recurrent product of that step, dz_t W_hh, as K-split
//               partial sums on the matrix cores (summed by the next step)
//   k_bwd_dh0   the last partial sums -> dh0
//   k_transpose, k_hprev_t, k_rowsum, k_cast_*  operand preparation for the
//               weight and input gradients, which are plain fp32 "NT" GEMMs
//               on the projection kernels
//   k_dropout_fwd, k_dropout_bwd  training dropout between layers: the trace
//               page's Performance Notes apply it to the input of every
//               layer above the first in training only; the draw is
//               Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
//               numbers: as easy as 1, 2, 3", SC 2011)
#include "device.h"
#include "kernels.h"

namespace lstm_amd {

// One backward step for every (direction, batch row, unit).  sb counts the
// backward steps: sb = 0 is the last step of each direction's scan.
__global__ void k_bwd_cell(BwdCellArgs a) {
    const size_t n = (size_t)a.D * a.B * a.H;
    const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int j = (int)(i % a.H);
    const int b = (int)((i / a.H) % a.B);
    const int d = (int)(i / ((size_t)a.H * a.B));
    const int T = a.T, B = a.B, H = a.H, D = a.D;
    const int sf = T - 1 - a.sb;                 // the forward scan's step
    const int t = d == 0 ? sf : T - 1 - sf;      // its time index
    const int tp = d == 0 ? t - 1 : t + 1;       // time of the scan's previous step
    const size_t dbj = ((size_t)d * B + b) * H + j;

    float dh = a.dY[((size_t)t * B + b) * ((size_t)D * H) + (size_t)d * H + j];
    float dcn;
    if (a.sb == 0) {
        dh += a.dhn ? a.dhn[dbj] : 0.f;
        dcn = a.dcn ? a.dcn[dbj] : 0.f;
    } else {
        // h_t feeds the next step's products: their partial sums, in slice
        // order, four loads in flight
        const float *pp = a.part + dbj;
        float r = 0.f;
        int p = 0;
        for (; p + 4 <= a.NP; p += 4) {
            const float v0 = pp[(size_t)p * n], v1 = pp[(size_t)(p + 1) * n];
            const float v2 = pp[(size_t)(p + 2) * n], v3 = pp[(size_t)(p + 3) * n];
            r += v0;
            r += v1;
            r += v2;
            r += v3;
        }
        for (; p < a.NP; ++p) r += pp[(size_t)p * n];
        dh += r;
        dcn = a.dc[dbj];
    }
    const float *ap = a.acts + (((size_t)t * B + b) * D + d) * 5 * H + j;
    const float ig = ap[0], fg = ap[(size_t)H], gg = ap[(size_t)2 * H], og = ap[(size_t)3 * H];
    const float c = ap[(size_t)4 * H];
    const float cprev = sf == 0 ? (a.c0 ? a.c0[dbj] : 0.f)
                                : a.acts[(((size_t)tp * B + b) * D + d) * 5 * H + (size_t)4 * H + j];
    const float tc = tanh_f(c);
    const float dct = dcn + dh * og * (1.f - tc * tc);
    float *dz = a.dz + (((size_t)t * B + b) * D + d) * 4 * H + j;
    dz[0] = dct * gg * ig * (1.f - ig);
    dz[(size_t)H] = dct * cprev * fg * (1.f - fg);
    dz[(size_t)2 * H] = dct * ig * (1.f - gg * gg);
    dz[(size_t)3 * H] = dh * tc * og * (1.f - og);
    a.dc[dbj] = dct * fg;
}

// part[p][d][b][j] = sum over k in slice p of dz_t[b][d][k] * W_hh[d][k][j]
// (K = 4H in the stacked gate order), with whT[d][j][k] = W_hh[d][k][j].
// A workgroup: 32 batch rows x 32 units of one direction and one K slice;
// wave (wm, wn) computes a 16 x 16 tile with 16x16x4 fp32 MFMAs whose
// fragments are 16-byte loads of K-contiguous rows.
__global__ __launch_bounds__(256) void k_bwd_mm(BwdMmArgs a) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w & 1, wn = w >> 1;
    const int B = a.B, H = a.H, D = a.D, K = 4 * H;
    const int p = blockIdx.z % a.NP, d = blockIdx.z / a.NP;
    const int b = blockIdx.x * 32 + wm * 16 + (lane & 15);  // A row of this lane
    const int j = blockIdx.y * 32 + wn * 16 + (lane & 15);  // B row (unit) of this lane
    const int k_lo = p * a.KS, k_hi = min(K, k_lo + a.KS);
    const int sf = a.T - 1 - a.sb;
    const int t = d == 0 ? sf : a.T - 1 - sf;
    // A: dz rows (t, b, d) for b < B; B: whT rows (d, j) for j < H.  Both via
    // buffer resources: a row past B or H, or a chunk past the slice, gets an
    // out-of-range offset and reads zeros without a memory access.
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.dz + ((size_t)t * B * D + d) * (size_t)K), (short)0,
        (int)(((size_t)(B - 1) * D * K + K) * sizeof(float)), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a.whT + (size_t)d * H * K), (short)0, (int)((size_t)H * K * sizeof(float)), 0x00020000);
    const unsigned aoff = (unsigned)((size_t)b * D * K * sizeof(float));
    const unsigned boff = (unsigned)((size_t)j * K * sizeof(float));
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // Batches of 16 chunks (a 256-deep slice is one batch): all 32 fragment
    // loads are issued before the first product of the batch, and a
    // scheduling barrier keeps the compiler from interleaving them with the
    // products into a chain of round trips (K % 4 == 0 and slices start at
    // multiples of 16: a fragment is whole or absent).
    constexpr int NBAT = 16;
    constexpr unsigned OOR = 0x7FFFFFF0u;
    for (int k0 = k_lo; k0 < k_hi; k0 += NBAT * F32::KC) {
        u32x4 av[NBAT], bv[NBAT];
#pragma unroll
        for (int c = 0; c < NBAT; ++c) {
            const int k = k0 + c * F32::KC + (lane >> 4) * F32::PER16;
            const bool kin = k < k_hi;
            av[c] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(kin && b < B ? aoff + 4u * k : OOR), 0, 0);
            bv[c] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(kin && j < H ? boff + 4u * k : OOR), 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < NBAT; ++c) acc = mma_chunk(F32{}, acc, av[c], bv[c]);
        __builtin_amdgcn_sched_barrier(0);
    }
    const size_t n = (size_t)D * B * H;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = blockIdx.x * 32 + wm * 16 + 4 * (lane >> 4) + v;
        const int u = blockIdx.y * 32 + wn * 16 + (lane & 15);
        if (m < B && u < H) a.part[(size_t)p * n + ((size_t)d * B + m) * H + u] = acc[v];
    }
}

// dh0 = the recurrent product of the scan's first step (sum of its partials)
template <class DT>
__global__ void k_bwd_dh0(const float *part, int NP, size_t n, typename DT::S *dh0) {
    const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    if (i >= n) return;
    float r = 0.f;
    for (int p = 0; p < NP; ++p) r += part[(size_t)p * n + i];
    dh0[i] = DT::from_f(r);
}

// out[c * ld_out + r] = in[r * ld_in + c] for r < rows, c < cols (as fp32)
template <class DT>
__global__ void k_transpose(const typename DT::S *in, size_t ld_in, int rows, int cols, float *out, size_t ld_out) {
    __shared__ float tile[32][33];
    const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
    for (int rr = threadIdx.y; rr < 32; rr += 8) {
        const int r = r0 + rr, c = c0 + threadIdx.x;
        tile[rr][threadIdx.x] = (r < rows && c < cols) ? DT::to_f(in[(size_t)r * ld_in + c]) : 0.f;
    }
    __syncthreads();
    for (int cc = threadIdx.y; cc < 32; cc += 8) {
        const int c = c0 + cc, r = r0 + threadIdx.x;
        if (c < cols && r < rows) out[(size_t)c * ld_out + r] = tile[threadIdx.x][cc];
    }
}

// out[k][m] = h_prev of direction d for row m = t*B + b (k < H, m < T*B):
// the layer's output at the time of the scan's previous step, or h0 (NULL =
// zeros) at the scan's first step.
template <class DT>
__global__ void k_hprev_t(const typename DT::S *Y, size_t ldy, const typename DT::S *h0d, int T, int B, int H,
                          int d, float *out) {
    __shared__ float tile[32][33];
    const int m0 = blockIdx.x * 32, k0 = blockIdx.y * 32;
    const int M = T * B;
    for (int mm = threadIdx.y; mm < 32; mm += 8) {
        const int m = m0 + mm, k = k0 + threadIdx.x;
        float v = 0.f;
        if (m < M && k < H) {
            const int t = m / B, b = m % B;
            const int tp = d == 0 ? t - 1 : t + 1;
            if (tp >= 0 && tp < T) v = DT::to_f(Y[((size_t)tp * B + b) * ldy + (size_t)d * H + k]);
            else if (h0d) v = DT::to_f(h0d[(size_t)b * H + k]);
        }
        tile[mm][threadIdx.x] = v;
    }
    __syncthreads();
    for (int kk = threadIdx.y; kk < 32; kk += 8) {
        const int k = k0 + kk, m = m0 + threadIdx.x;
        if (k < H && m < M) out[(size_t)k * M + m] = tile[threadIdx.x][kk];
    }
}

// out[r] = sum over c of a[r * ld + c]: one workgroup per row, a fixed tree
// (deterministic)
__global__ void k_rowsum(const float *a, size_t ld, int cols, float *out) {
    __shared__ float red[256];
    const float *row = a + (size_t)blockIdx.x * ld;
    float s = 0.f;
    for (int c = threadIdx.x; c < cols; c += 256) s += row[c];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = red[0];
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
        for (int sp = 1; sp < ns; ++sp) v += part[(size_t)sp * slab + i];
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
                              float scale) {
    const size_t nblk = (n + 3) / 4;
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < nblk; i += (size_t)gridDim.x * blockDim.x) {
        unsigned long long c[4] = {(unsigned long long)i, (unsigned long long)layer, call, 0ull};
        philox4x64_10(c, seed, 0ull);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const size_t e = 4 * i + q;
            if (e >= n) break;
            const bool kept = (c[q] >> 11) >= thr;
            xd[e] = DT::from_f(kept ? DT::to_f(y[e]) * scale : 0.f);
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

hipError_t launch_bwd_cell(const BwdCellArgs &a, hipStream_t s) {
    const size_t n = (size_t)a.D * a.B * a.H;
    hipLaunchKernelGGL(k_bwd_cell, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bwd_mm(const BwdMmArgs &a, hipStream_t s) {
    if ((4 * a.H) % 4 != 0 || a.KS % F32::KC != 0) return hipErrorInvalidValue;
    dim3 grid((a.B + 31) / 32, (a.H + 31) / 32, a.NP * a.D);
    hipLaunchKernelGGL(k_bwd_mm, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bwd_dh0(const float *part, int NP, size_t n, void *dh0, int dtype, hipStream_t s) {
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(k_bwd_dh0<BF16>, dim3(grid1(n, 1u << 30)), dim3(256), 0, s, part, NP, n,
                           static_cast<uint16_t *>(dh0));
    else
        hipLaunchKernelGGL(k_bwd_dh0<F32>, dim3(grid1(n, 1u << 30)), dim3(256), 0, s, part, NP, n,
                           static_cast<float *>(dh0));
    return hipGetLastError();
}

hipError_t launch_transpose(const void *in, size_t ld_in, int rows, int cols, float *out, size_t ld_out, int dtype,
                            hipStream_t s) {
    dim3 grid((cols + 31) / 32, (rows + 31) / 32), block(32, 8);
    if (grid.y > 65535u) return hipErrorInvalidValue;
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(k_transpose<BF16>, grid, block, 0, s, static_cast<const uint16_t *>(in), ld_in, rows,
                           cols, out, ld_out);
    else
        hipLaunchKernelGGL(k_transpose<F32>, grid, block, 0, s, static_cast<const float *>(in), ld_in, rows, cols,
                           out, ld_out);
    return hipGetLastError();
}

hipError_t launch_hprev_t(const void *Y, size_t ldy, const void *h0d, int T, int B, int H, int d, float *out,
                          int dtype, hipStream_t s) {
    dim3 grid(((size_t)T * B + 31) / 32, (H + 31) / 32), block(32, 8);
    if (grid.y > 65535u) return hipErrorInvalidValue;
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(k_hprev_t<BF16>, grid, block, 0, s, static_cast<const uint16_t *>(Y), ldy,
                           static_cast<const uint16_t *>(h0d), T, B, H, d, out);
    else
        hipLaunchKernelGGL(k_hprev_t<F32>, grid, block, 0, s, static_cast<const float *>(Y), ldy,
                           static_cast<const float *>(h0d), T, B, H, d, out);
    return hipGetLastError();
}

hipError_t launch_rowsum(const float *a, size_t ld, int rows, int cols, float *out, hipStream_t s) {
    if (rows < 1) return hipSuccess;
    hipLaunchKernelGGL(k_rowsum, dim3(rows), dim3(256), 0, s, a, ld, cols, out);
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

hipError_t launch_dropout_fwd(const void *y, void *xd, unsigned char *keep, size_t n, unsigned long long seed,
                              unsigned long long call, int layer, unsigned long long thr, float scale, int dtype,
                              hipStream_t s) {
    if (n == 0) return hipSuccess;
    const unsigned g = grid1((n + 3) / 4);
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(k_dropout_fwd<BF16>, dim3(g), dim3(256), 0, s, static_cast<const uint16_t *>(y),
                           static_cast<uint16_t *>(xd), keep, n, seed, call, layer, thr, scale);
    else
        hipLaunchKernelGGL(k_dropout_fwd<F32>, dim3(g), dim3(256), 0, s, static_cast<const float *>(y),
                           static_cast<float *>(xd), keep, n, seed, call, layer, thr, scale);
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
