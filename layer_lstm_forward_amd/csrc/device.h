// device.h -- device-side building blocks shared by the gfx950 kernels:
// element traits, 16-byte fragment loads, MFMA chunk products, the gate
// nonlinearities and the cross-workgroup step barrier.
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

// sigma(z) = 1 / (1 + e^-z) from the hardware base-2 exponential and
// reciprocal; exp2 overflows to +inf for very negative z and the reciprocal
// of +inf is 0, so the saturated ends are exact.  tanh(z) = 2 sigma(2z) - 1.
__device__ inline float sigmoid_f(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}
__device__ inline float tanh_f(float z) { return 2.0f * sigmoid_f(2.0f * z) - 1.0f; }

// ---------------------------------------------------------------------------
// Step barrier between the workgroups that exchange one direction's hidden
// state.  Each workgroup adds 1 to its team counter after publishing a step;
// a consumer waits until the counter reaches (members * steps).  Counters only
// grow within one launch, so no reset is needed between steps.
//
// Memory ordering: every thread that stored part of h_t issues an agent-scope
// release fence before the workgroup barrier, and thread 0 then bumps the
// counter; the waiting side observes the counter with agent-scope loads and
// every thread issues an agent-scope acquire fence before reading h_t.
//
// The wait is bounded in wall-clock time: on expiry it raises bit 0 of the
// status word and every waiter leaves, so a launch always drains.
// ---------------------------------------------------------------------------
__device__ inline void step_publish(unsigned *ctr) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline bool step_wait(const unsigned *ctr, unsigned target, unsigned *status,
                                 long long timeout_ticks, int *s_flag) {
    if (threadIdx.x == 0) {
        int ok = 1;
        unsigned it = 0;
        const long long t0 = wall_clock64();
        while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if ((++it & 127u) == 0) {
                if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
                    ok = 0;
                    break;
                }
                if (wall_clock64() - t0 > timeout_ticks) {
                    __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    ok = 0;
                    break;
                }
            }
            __builtin_amdgcn_s_sleep(1);
        }
        *s_flag = ok;
    }
    __syncthreads();
    const int ok = *s_flag;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return ok != 0;
}

}  // namespace lstm_amd
