// noalloc.hip -- lstm_forward_static: lstm_forward with its workspace in a
// file-scope device array of the library instead of caller memory, for
// callers that cannot allocate device memory (include/lstm.h).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/lstm.h"
#include "kernels.h"

namespace {

// The workspace of lstm_forward_static.  Each device the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: its
// device address comes from scratch_address().
static __device__ __align__(256) unsigned char scratch[LSTM_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // the address of `scratch` on each device (nullptr: not looked up yet)

// The address of `scratch` on the current device, looked up on the first
// call made with that device current and kept.
lstm_status scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices) return LSTM_ERR_DEVICE;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return LSTM_ERR_DEVICE;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return LSTM_OK;
}

bool is_device_memory(const void *ptr) {
    int dev = 0;
    hipPointerAttribute_t attr{};
    if (hipGetDevice(&dev) != hipSuccess || hipPointerGetAttributes(&attr, ptr) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) && attr.device == dev;
}

// *dst = *src, the status word at the start of the workspace
__global__ void k_copy_status(unsigned *dst, const unsigned *src) {
    if (threadIdx.x == 0) *dst = *src;
}

}  // namespace

extern "C" lstm_status lstm_forward_static(lstm_plan *p, const void *x, const void *h0, const float *c0,
                                           const void *const *weights, int T, int B, int layers, int bidir,
                                           void *y, void *h_n, float *c_n, unsigned *device_status,
                                           void *stream) {
    if (!p) return LSTM_ERR_ARG;
    size_t need = 0;
    lstm_status rc = lstm_workspace_size(p, T, B, &need);
    if (rc != LSTM_OK) return rc;
    if (need > LSTM_STATIC_WORKSPACE_BYTES) return LSTM_ERR_WORKSPACE;
    if (device_status && !is_device_memory(device_status)) return LSTM_ERR_DEVICE;
    void *ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != LSTM_OK) return rc;
    rc = lstm_amd::forward_dispatch(p, x, h0, c0, weights, T, B, layers, bidir, y, h_n, c_n, ws,
                                    LSTM_STATIC_WORKSPACE_BYTES, stream, true);
    if (rc != LSTM_OK || !device_status) return rc;
    hipLaunchKernelGGL(k_copy_status, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), device_status,
                       static_cast<const unsigned *>(ws));
    if (hipGetLastError() != hipSuccess) return LSTM_ERR_LAUNCH;
    return LSTM_OK;
}
