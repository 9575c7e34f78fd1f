// Row moves between PyTorch's packed-sequence layout and the padded
// time-major layout the forward runs on.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>

namespace lstm_amd {

// gather (to_padded): dst row map[r] = src row r; else dst row r = src row
// map[r]; r < n, rows of row_bytes bytes (a multiple of 2).  Rows of the
// padded side that no r names are left as they are.
hipError_t launch_copy_rows(const void *src, void *dst, const int *map, int n, size_t row_bytes, bool to_padded,
                            hipStream_t s);

}  // namespace lstm_amd
