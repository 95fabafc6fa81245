// Allocation-free decode: dsv4_sparse_decode with its split partials in a
// fixed device array of this library (`scratch`) instead of a caller's
// workspace, for callers that cannot allocate device memory.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, from the loading of the code
// object to the end of the process.  In host code `scratch` names a host-side
// stand-in, never the device memory, so its device address is taken once per
// device, with that device current, through hipGetSymbolAddress, and only
// that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "dsv4.h"
#include "internal.hpp"

namespace {

constexpr size_t kScratchBytes = DSV4_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];   // device address of `scratch`, per device
std::mutex g_scratch_mu;

// Device address of this device's `scratch`, looked up on the first call
// made with the device current.
int scratch_address(int dev, void** out) {
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return dsv4::set_last_error(DSV4_ERR_HIP,
                                            "hipGetSymbolAddress(scratch) on device %d failed: %s",
                                            dev, hipGetErrorString(e));
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return DSV4_OK;
}

}  // namespace

extern "C" int dsv4_sparse_decode_noalloc(const dsv4_decode_desc* desc, const void* q,
                                          const void* kv_cache, const int32_t* block_table,
                                          const int32_t* topk_idx, const int32_t* valid_len,
                                          const float* sink, void* out, float* lse,
                                          int32_t num_splits, hipStream_t stream) {
    dsv4_plan plan;
    const int st = dsv4_sparse_decode_plan(desc, num_splits, &plan);
    if (st) return st;
    if (plan.workspace_bytes > kScratchBytes)
        return dsv4::set_last_error(
            DSV4_ERR_WORKSPACE_TOO_SMALL,
            "this decode (batch %d, %d heads, %d splits) needs %zu bytes of split partials; the "
            "allocation-free entry point holds at most %zu (DSV4_NOALLOC_SCRATCH_BYTES): use "
            "dsv4_sparse_decode with a workspace, or fewer splits",
            desc->batch, desc->num_heads, plan.num_splits, plan.workspace_bytes,
            (size_t)kScratchBytes);
    dsv4_decode_desc d = *desc;
    d.workspace = nullptr;
    d.workspace_bytes = 0;
    if (plan.workspace_bytes) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return dsv4::set_last_error(DSV4_ERR_HIP, "hipGetDevice failed: %s",
                                        hipGetErrorString(e));
        if (stream) {
            int sdev = dev;
            e = hipStreamGetDevice(stream, &sdev);
            if (e != hipSuccess)
                return dsv4::set_last_error(DSV4_ERR_HIP, "hipStreamGetDevice failed: %s",
                                            hipGetErrorString(e));
            if (sdev != dev)
                return dsv4::set_last_error(
                    DSV4_ERR_INVALID_ARGUMENT,
                    "the stream belongs to device %d but device %d is current", sdev, dev);
        }
        if (dev < 0 || dev >= kMaxDevices)
            return dsv4::set_last_error(DSV4_ERR_NOT_SUPPORTED, "device %d: at most %d devices",
                                        dev, kMaxDevices);
        void* p = nullptr;
        const int s2 = scratch_address(dev, &p);
        if (s2) return s2;
        d.workspace = p;
        d.workspace_bytes = kScratchBytes;
    }
    return dsv4_sparse_decode(&d, q, kv_cache, block_table, topk_idx, valid_len, sink, out, lse,
                              num_splits, stream);
}
