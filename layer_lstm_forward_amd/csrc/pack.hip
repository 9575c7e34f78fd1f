// Packed sequences (the trace page "Complete Trace: nn.LSTM", Step 3: the
// overload that takes data and batch_sizes): the rows of step t are rows
// offset_t .. offset_t + batch_sizes[t] - 1 of the packed data, one per
// sequence still running at t.  The forward runs on the padded time-major
// layout; these kernels move whole rows between the two by a row map.
#include "pack.h"

namespace lstm_amd {

// One workgroup per row (grid-stride over rows); 16-byte moves when the row
// and both bases allow them, else 2-byte ones.
template <class V>
__global__ void k_copy_rows(const char *src, char *dst, const int *map, int n, size_t row_bytes, int to_padded) {
    const size_t nv = row_bytes / sizeof(V);
    for (int r = blockIdx.x; r < n; r += gridDim.x) {
        const size_t pr = (size_t)map[r];
        const V *s = reinterpret_cast<const V *>(src + (to_padded ? (size_t)r : pr) * row_bytes);
        V *d = reinterpret_cast<V *>(dst + (to_padded ? pr : (size_t)r) * row_bytes);
        for (size_t i = threadIdx.x; i < nv; i += blockDim.x) d[i] = s[i];
    }
}

hipError_t launch_copy_rows(const void *src, void *dst, const int *map, int n, size_t row_bytes, bool to_padded,
                            hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (row_bytes % 2 != 0) return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)(n < 65536 ? n : 65536);
    const bool v16 = row_bytes % 16 == 0 && (uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0;
    if (v16)
        hipLaunchKernelGGL(k_copy_rows<uint4>, dim3(blocks), dim3(128), 0, s, static_cast<const char *>(src),
                           static_cast<char *>(dst), map, n, row_bytes, to_padded ? 1 : 0);
    else
        hipLaunchKernelGGL(k_copy_rows<unsigned short>, dim3(blocks), dim3(128), 0, s,
                           static_cast<const char *>(src), static_cast<char *>(dst), map, n, row_bytes,
                           to_padded ? 1 : 0);
    return hipGetLastError();
}

}  // namespace lstm_amd
