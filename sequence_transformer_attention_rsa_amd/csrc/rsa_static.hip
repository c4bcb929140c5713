// rsa_static.hip -- the backward entry point that allocates nothing.
//
// rsa_backward needs a workspace for its row statistics (8 bytes per query
// row), which the caller allocates. Callers that cannot allocate device
// memory at the point of the call (code under HIP graph capture, serving
// loops that must not allocate, harnesses that forbid it) call
// rsa_backward_noalloc instead: the row statistics then live in `scratch`,
// a fixed array in device memory that every GPU the library runs on holds
// until the process ends.
//
// `scratch` is a device symbol: in host code its name is a host-side
// stand-in, not a device address. Its address on a device is resolved once
// per device, with that device current, by hipGetSymbolAddress, and only
// that address is ever passed to a kernel. Every call on one GPU shares the
// array: calls that overlap on one GPU (two streams, two threads) race.
// Nothing in it needs clearing between calls: the first stage of the
// backward writes every row statistic that the later stages read.

#include <mutex>

#include <hip/hip_runtime.h>

#include "rsa.h"
#include "rsa_internal.h"

namespace {

constexpr size_t kScratchBytes = RSA_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device, once resolved

// The device whose memory the stream's work uses (the current device for the
// null stream).
hipError_t stream_device(hipStream_t stream, int* dev) {
    if (stream == nullptr) return hipGetDevice(dev);
    return hipStreamGetDevice(stream, dev);
}

// Device address of `scratch` on the stream's device, resolved on the first
// call for that device with the device current (the caller's current device
// is restored afterwards).
int scratch_address(hipStream_t stream, void** out) {
    int dev = -1;
    if (stream_device(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RSA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return RSA_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return RSA_ERR_HIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr) return RSA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return RSA_OK;
}

}  // namespace

extern "C" int rsa_backward_noalloc(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                    const float* lse, const uint8_t* key_mask,
                                    int B, int H, int L, int d, int N, int dtype, int flags,
                                    void* stream, void* dq, void* dk, void* dv) {
    // every check but the workspace's, before any HIP call
    int st = rsa::check_backward_call(q, k, v, out, dout, lse, key_mask, B, H, L, d, N, dtype, flags, dq, dk, dv);
    if (st != RSA_OK) return st;
    if (rsa_backward_workspace_bytes(B, H, L, d, N, dtype) > kScratchBytes) return RSA_ERR_SCRATCH;
    void* ws = nullptr;
    st = scratch_address(static_cast<hipStream_t>(stream), &ws);
    if (st != RSA_OK) return st;
    return rsa_backward_ex(q, k, v, out, dout, lse, key_mask, B, H, L, d, N, dtype, flags, ws, kScratchBytes, stream,
                           dq, dk, dv);
}
