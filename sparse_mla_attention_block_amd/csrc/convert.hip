// Req-local -> global slot conversion through a block table (vLLM PR #41217
// report, key source snippets: the req-index to global-index kernel, with
// its block range check, invalid fill and ragged store from seq_start).
// Differences from that kernel: the fill value is an argument, a negative
// page entry or an unrepresentable slot also yields the fill, requests
// outside the table are filled instead of read, and columns past the row
// width are never loaded.
//
// One lane per output element; grid.x = tokens, grid.y = 256-column tiles
// (at most 65535 of them: a row wider than 65535 x 256 columns is walked in
// strides of the grid's columns).  Integer work only, so the result is
// bit-exact by construction.
#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace dsv4 {

constexpr int kConvertThreads = 256;

__global__ __launch_bounds__(kConvertThreads) void convert_kernel(const ConvertParams p) {
    const int t = blockIdx.x;
    int64_t base, n;
    if (p.cu) {
        base = p.cu[t];
        n = (int64_t)p.cu[t + 1] - p.cu[t];
        if (n > p.width) n = p.width;
    } else {
        base = (int64_t)t * p.width;
        n = p.width;
    }
    const int32_t req = p.req_id ? p.req_id[t] : p.sq == 1 ? t : t / p.sq;
    const int64_t stride = (int64_t)gridDim.y * kConvertThreads;
    for (int64_t i = (int64_t)blockIdx.y * kConvertThreads + threadIdx.x; i < n; i += stride) {
        // Positions outside [0, cu[num_tokens]) are never written, whatever cu holds.
        if (p.cu && (base + i < 0 || base + i >= p.cu[p.num_tokens])) continue;
        const int32_t idx = p.ti[(int64_t)t * p.ti_stride + i];
        int64_t v = p.fill;
        if (idx >= 0 && req >= 0 && req < p.num_reqs) {
            const int64_t blk = idx / p.bs;
            const int64_t off = idx % p.bs;
            if (blk < p.max_blocks) {
                const int64_t page = p.bt[(int64_t)req * p.bt_stride + blk];
                if (page >= 0) {
                    const int64_t gslot = page * p.bs + off;
                    if (gslot <= 2147483647LL) v = gslot;
                }
            }
        }
        p.out[base + i] = (int32_t)v;
    }
}

hipError_t launch_convert(const ConvertParams& p, hipStream_t stream) {
    int64_t tiles = ((int64_t)p.width + kConvertThreads - 1) / kConvertThreads;
    if (tiles > 65535) tiles = 65535;
    const dim3 grid((unsigned)p.num_tokens, (unsigned)tiles);
    hipLaunchKernelGGL(convert_kernel, grid, dim3(kConvertThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace dsv4
