// device.h -- device-side building blocks shared by the gfx950 kernels:
// element traits, 16-byte fragment loads, MFMA chunk products, the gate
// nonlinearities and the tagged hidden-state exchange between workgroups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lstm_amd {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Element traits.  A "fragment" is the 16 bytes one lane feeds to the matrix
// core per chunk; a "chunk" is the K extent that 64 lanes x 16 bytes cover for
// a 16-row tile: 16 fp32 values (four v_mfma_f32_16x16x4_f32) or 32 bf16
// values (one v_mfma_f32_16x16x32_bf16).  Lane l holds row (l % 16) and the
// K sub-range (l / 16) * PER16 .. + PER16 - 1 of the chunk, for both operands,
// so every chunk product sums over exactly the chunk's K range.
struct F32 {
    using S = float;                 // storage type
    static constexpr int PER16 = 4;  // elements per 16-byte fragment
    static constexpr int KC = 16;    // K per chunk
    __device__ static float to_f(S v) { return v; }
    __device__ static S from_f(float v) { return v; }
};
struct BF16 {
    using S = uint16_t;              // bfloat16 bit pattern
    static constexpr int PER16 = 8;
    static constexpr int KC = 32;
    __device__ static float to_f(S v) { return __uint_as_float((uint32_t)v << 16); }
    // round to nearest, ties to even (values here are finite)
    __device__ static S from_f(float v) {
        uint32_t u = __float_as_uint(v);
        u += 0x7FFFu + ((u >> 16) & 1u);
        return (S)(u >> 16);
    }
};

// acc += A_chunk * B_chunk^T for one 16x16 output tile.
__device__ inline f32x4 mma_chunk(F32, f32x4 acc, u32x4 a, u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
    return acc;
}
__device__ inline f32x4 mma_chunk(BF16, f32x4 acc, u32x4 a, u32x4 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// acc += A * B^T for one 32x32 output tile over 32 bytes of K per row: lane l
// feeds row (l % 32) with K sub-range (l / 32) * PER16 .. + PER16 - 1; the
// result lane l, register v holds row 8*(v/4) + 4*(l/32) + v%4, column l%32.
__device__ inline f32x16 mma32_chunk(F32, f32x16 acc, u32x4 a, u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
    return acc;
}
__device__ inline f32x16 mma32_chunk(BF16, f32x16 acc, u32x4 a, u32x4 b) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   acc, 0, 0, 0);
}

// Load the 16-byte fragment row[k .. k+PER16) with zero fill past kmax.
// vec: the caller guarantees 16-byte alignment of row + k whenever the whole
// fragment is in range.
template <class DT>
__device__ inline u32x4 load_frag(const typename DT::S *row, int k, int kmax, bool vec) {
    using S = typename DT::S;
    if (vec && k + DT::PER16 <= kmax) return *reinterpret_cast<const u32x4 *>(row + k);
    S tmp[DT::PER16];
#pragma unroll
    for (int e = 0; e < DT::PER16; ++e) tmp[e] = (k + e < kmax) ? row[k + e] : (S)0;
    return __builtin_bit_cast(u32x4, tmp);
}

// Row of (time t, batch b) in x, G and y: time-major [T][B] rows, or
// batch-major [B][T] rows (batch_first).
__device__ inline size_t trow(int t, int b, int T, int B, bool batch_first) {
    return batch_first ? (size_t)b * T + t : (size_t)t * B + b;
}

// sigma(z) = 1 / (1 + e^-z) from the hardware base-2 exponential and
// reciprocal; exp2 overflows to +inf for very negative z and the reciprocal
// of +inf is 0, so the saturated ends are exact.  tanh(z) = 2 sigma(2z) - 1.
__device__ inline float sigmoid_f(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}
__device__ inline float tanh_f(float z) { return 2.0f * sigmoid_f(2.0f * z) - 1.0f; }

// ---------------------------------------------------------------------------
// Hidden-state exchange between workgroups.  h_t travels as 64-bit words whose
// high half is a step tag and whose low half carries the value (one fp32, or
// two bf16 of adjacent units).  Producers store them with agent-scope atomic
// stores and consumers read them with agent-scope atomic loads; on gfx950 both
// are single 64-bit accesses performed at the device coherence point (the
// "sc1" scope bits), so a word is seen either whole-old or whole-new, from any
// XCD, without cache write-back or invalidation.  A consumer simply re-reads
// each word until it carries the tag it expects: the arrival of the data is
// the synchronisation, and no counter or barrier is involved.
// ---------------------------------------------------------------------------
__device__ inline unsigned long long xload(const unsigned long long *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void xstore(unsigned long long *p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned long long xword(unsigned tag, uint32_t payload) {
    return ((unsigned long long)tag << 32) | payload;
}
__device__ inline unsigned xtag(unsigned long long w) { return (unsigned)(w >> 32); }

// Two adjacent tagged words in one 16-byte agent-scope ("sc1") buffer load.
// Each 8-byte word carries its own tag, so only 8-byte single-copy atomicity
// of the halves is relied on.  Offsets at or past the resource size return
// zeros without a memory access.
__device__ inline __amdgpu_buffer_rsrc_t xrsrc(const unsigned long long *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned long long *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ inline u32x4 xload2(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 16 /* sc1: device scope */);
}

// ---------------------------------------------------------------------------
// Compact exchange words (the per-layer recurrence).  A 32-bit word carries
// the value and a one-bit step tag, stored with an agent-scope atomic 32-bit
// store and read (four words at a time) with the 16-byte sc1 load above; each
// word is a single-copy atomic unit.  Three word formats:
//   fp32:      one value; the tag is the least significant mantissa bit.  The
//              value a consumer multiplies is h or its fp32 neighbour (at most
//              1 ulp away); NaN stays NaN.  Any h.
//   bf16 pair: two bf16 values of adjacent units (low half: the even unit);
//              the tag is bit 30, the top exponent bit of the upper value.
//              That bit is clear in the value itself only while |h| < 2 (a
//              bf16 of magnitude >= 2 has a biased exponent >= 128), so this
//              format is only for values bounded by 1: the LSTM's o tanh(c)
//              and the tanh RNN's output.  A non-finite h is sent as a NaN in
//              the lower half (the batch row becomes NaN at the next step
//              either way, as it would with the true value).
//   bf16 wide: one bf16 value in the upper half, the tag in bit 0 (the word
//              is the value's exact fp32 form plus the tag in a bit that is
//              zero in every bf16).  Any h, at twice the bytes of the pair
//              format: used wherever a published h may reach 2 in magnitude
//              (the relu RNN, the GRU started from a caller's h0, and padded
//              steps that republish a caller's h0).
// One bit suffices because each location is written once every two steps
// and each consumer lane always reads the same locations: the value it last
// accepted there was the previous write, and read-read coherence of a
// location forbids it from seeing anything older afterwards, so the only
// values it can observe are the previous write (tag differs) or the current
// one.  The host keeps the tag sequence continuous across the layers of a
// call (the buffer is zeroed once per call, and a zero word carries tag 0).
// The word functions are host-callable so that the formats can be checked on
// the CPU.
// ---------------------------------------------------------------------------
enum XFmt { XF_F32 = 0, XF_PAIR = 1, XF_WIDE = 2 };
// bit position of the tag in a word of format f
__host__ __device__ constexpr unsigned xc_shift(int f) { return f == XF_PAIR ? 30u : 0u; }
__host__ __device__ inline uint32_t xc_word_f32(uint32_t hbits, unsigned tb) { return (hbits & ~1u) | tb; }
__host__ __device__ inline uint32_t xc_word_pair(uint16_t lo, uint16_t hi, unsigned tb) {
    const bool nonfinite = ((lo & 0x7F80u) == 0x7F80u) || ((hi & 0x7F80u) == 0x7F80u);
    const uint32_t payload = nonfinite ? 0x7FC0u : ((uint32_t)lo | ((uint32_t)hi << 16));
    return payload | (tb << 30);
}
__host__ __device__ inline uint32_t xc_word_wide(uint16_t h, unsigned tb) { return ((uint32_t)h << 16) | tb; }
// the tag bit a word of format f carries
__host__ __device__ inline unsigned xc_word_tag(uint32_t w, int f) { return (w >> xc_shift(f)) & 1u; }
// the value bits of a pair word with its tag removed (two bf16)
__host__ __device__ inline uint32_t xc_pair_value(uint32_t w) { return w & 0xBFFFFFFFu; }
// two wide words (values e and e + 1) as one bf16 pair, value e in the low half
__host__ __device__ inline uint32_t xc_wide_pair(uint32_t w0, uint32_t w1) {
    return (w0 >> 16) | (w1 & 0xFFFF0000u);
}
__device__ inline void xcstore(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline __amdgpu_buffer_rsrc_t xcrsrc(const uint32_t *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(base), (short)0, (int)bytes, 0x00020000);
}
// tag bit of the write made at step s into buffer s & 1
__host__ __device__ inline unsigned xc_tag(unsigned xpar, int s) {
    return (((xpar >> (s & 1)) & 1u) + ((unsigned)s >> 1) + 1u) & 1u;
}
// all four words of a 16-byte load carry tag bit tb
template <int F>
__host__ __device__ inline bool xc_ok(const u32x4 &w, unsigned tb) {
    const unsigned all = w.x & w.y & w.z & w.w, any = w.x | w.y | w.z | w.w;
    return ((tb ? all : ~any) >> xc_shift(F)) & 1u;
}

// Sum of the N f32x4 partial sums at p, p + stride, ..., p + (N-1) stride
// (floats, in LDS), added in index order.  All N reads are issued before the
// first addition, so the reduction costs one LDS round trip, not N.
template <int N>
__device__ inline f32x4 lds_sum_f32x4(const float *p, int stride) {
    f32x4 v[N];
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = *reinterpret_cast<const f32x4 *>(p + k * stride);
    f32x4 sum = v[0];
#pragma unroll
    for (int k = 1; k < N; ++k) sum += v[k];
    return sum;
}

// The float at byte offset off of a buffer of nbytes bytes, through a buffer
// resource: a NULL base (no records) reads 0, without a branch (a branch
// around a load makes the compiler wait for it where the paths join).
__device__ inline float load_f32_or0(const void *base, unsigned nbytes, unsigned off) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                                                       base ? (int)nbytes : 0, 0x00020000);
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// The same for an element of the storage type of DT (bf16 or fp32), widened.
template <class DT>
__device__ inline float load_s_or0(const void *base, unsigned nbytes, unsigned off) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                                                       base ? (int)nbytes : 0, 0x00020000);
    if constexpr (sizeof(typename DT::S) == 2)
        return DT::to_f((typename DT::S)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
    else
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

}  // namespace lstm_amd
