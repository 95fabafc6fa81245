// Cache writer: quantise bf16 rows and store them into fp8_ds_mla pages
// (vLLM PR #52212 page, the sanitising writer snippet: UE8M0 codes clamped
// to [0, 254] and non-finite RoPE values stored as 0 when sanitising,
// [0, 255] and RoPE untouched otherwise).  The amax -> code step is not on
// the pages; the code taken is the smallest one whose scale brings the
// group's largest magnitude within the E4M3FN range (|v| <= 448).
//
// Each wave quantises 2 consecutive rows (8 per workgroup), one at a time
// after loading both.  Lane l holds dims [8l, 8l+8) of a row:
// lanes 0..55 the seven 64-dim NoPE groups (8 lanes each), lanes 56..63 the
// RoPE dims.  The group maximum is taken on bf16 magnitude bits (integer
// order equals magnitude order; NaN is dropped first), so the code is exact
// integer arithmetic; scaling by 2^(127-c) is exact; the E4M3FN rounding is
// the hardware convert of values already clamped to [-448, 448].  Input rows
// and cache bytes are each touched once, so loads and stores are
// nontemporal (streaming: 3-6 % faster than cached accesses).
#include <hip/hip_runtime.h>

#include "device_util.hpp"
#include "internal.hpp"

namespace dsv4 {

constexpr int kStoreThreads = 256;
constexpr int kStoreRowsPerWave = 2;
constexpr int kStoreRows = kStoreThreads / 64 * kStoreRowsPerWave;   // per workgroup

// Smallest UE8M0 code c with a <= 448 * 2^(c-127) for the bf16 magnitude
// bits a (NaN excluded), clamped to [0, cap].  With a = (1 + M/128) 2^(E-127)
// and 448 = 1.75 * 2^8: c = E - 8 when M/128 <= 0.75, else E - 7; an
// infinity has no such code and takes the cap.
__device__ __forceinline__ int ue8m0_code(uint32_t a, int cap) {
    if (a >= 0x7F80u) return cap;
    const int c = (int)(a >> 7) - 8 + ((a & 0x7Fu) > 96u ? 1 : 0);
    return c < 0 ? 0 : (c > cap ? cap : c);
}

// Four bf16 (two words) -> four E4M3FN bytes scaled by 2^(127-c).
__device__ __forceinline__ uint32_t quant4(uint32_t w0, uint32_t w1, int c) {
    const int e = 127 - c;
    float y[4] = {__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xFFFF0000u),
                  __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xFFFF0000u)};
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = fminf(fmaxf(ldexpf(y[i], e), -448.0f), 448.0f);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], r, true);
    // NaN inputs store the E4M3FN NaN 0x7F whatever the convert made of them.
    const uint32_t h[4] = {w0 & 0x7FFFu, w0 >> 16 & 0x7FFFu, w1 & 0x7FFFu, w1 >> 16 & 0x7FFFu};
    uint32_t out = (uint32_t)r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (h[i] > 0x7F80u) out = (out & ~(0xFFu << (8 * i))) | (0x7Fu << (8 * i));
    return out;
}

// Quantises the row whose 8 bf16 values this lane holds and stores it at
// `slot` (a skipped slot stores nothing; the caller's branch is wave-uniform).
__device__ __forceinline__ void store_row(const StoreParams& p, int lane, int64_t slot,
                                          const uint4 in) {
    const uint32_t w[4] = {in.x, in.y, in.z, in.w};
    // Largest finite-or-infinite magnitude of the lane's 8 values, then of
    // its 8-lane group (xor 1, 2, 4 stay inside aligned groups of 8).
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] & 0x7FFFu, hi = w[i] >> 16 & 0x7FFFu;
        a = max(a, lo > 0x7F80u ? 0u : lo);
        a = max(a, hi > 0x7F80u ? 0u : hi);
    }
    a = max(a, (uint32_t)__shfl_xor((int)a, 1));
    a = max(a, (uint32_t)__shfl_xor((int)a, 2));
    a = max(a, (uint32_t)__shfl_xor((int)a, 4));
    const int c = ue8m0_code(a, p.sanitize ? 254 : 255);

    // Page and offset: 32-bit division when every slot fits in 32 bits (a
    // wave-uniform branch on the pool size), 64-bit otherwise.
    int64_t page, off;
    if (p.num_slots <= 0xFFFFFFFFll) {
        const uint32_t s32 = (uint32_t)slot, q = s32 / (uint32_t)p.bs;
        page = q;
        off = s32 - q * (uint32_t)p.bs;
    } else {
        page = slot / p.bs;
        off = slot - page * p.bs;
    }
    uint8_t* base = p.kv + page * p.page_stride;
    uint8_t* data = base + off * kRowData;
    if (lane < kDNope / 8) {
        {
            const uint64_t v64 = (uint64_t)quant4(w[2], w[3], c) << 32 | quant4(w[0], w[1], c);
            __builtin_nontemporal_store(v64, reinterpret_cast<uint64_t*>(data + 8 * lane));
        }
    } else {
        uint32_t v[4] = {w[0], w[1], w[2], w[3]};
        if (p.sanitize) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = scrub_pair(v[i]);
        }
        uint8_t* dst = data + kDNope + 16 * (lane - kDNope / 8);
        __builtin_nontemporal_store((uint64_t)v[1] << 32 | v[0],
                                    reinterpret_cast<uint64_t*>(dst));
        __builtin_nontemporal_store((uint64_t)v[3] << 32 | v[2],
                                    reinterpret_cast<uint64_t*>(dst + 8));
    }
    // Scale word: the seven group codes and a zero pad byte, stored by lane 0.
    uint64_t sw = 0;
#pragma unroll
    for (int g = 0; g < kDNope / 64; ++g)
        sw |= (uint64_t)(uint32_t)__builtin_amdgcn_readlane(c, 8 * g) << (8 * g);
    if (lane == 0)
        __builtin_nontemporal_store(
            sw, reinterpret_cast<uint64_t*>(base + (int64_t)p.bs * kRowData + off * kRowScale));
}

// Each wave takes kStoreRowsPerWave consecutive rows and issues all their
// loads before the first store, so that every wave keeps that many 1 KB
// rows in flight.
__global__ __launch_bounds__(kStoreThreads) void quantize_store_kernel(const StoreParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t row0 =
        ((int64_t)blockIdx.x * (kStoreThreads / 64) + (threadIdx.x >> 6)) * kStoreRowsPerWave;
    if (row0 >= p.n) return;                      // whole waves leave together
    uint4 in[kStoreRowsPerWave];
    int64_t slot[kStoreRowsPerWave];
#pragma unroll
    for (int i = 0; i < kStoreRowsPerWave; ++i) {
        const int64_t r = row0 + i < p.n ? row0 + i : p.n - 1;   // tail rows re-read the last
        // The slot is the same for the whole wave: keep it in scalar registers.
        const int64_t s_ld = p.slots[r];
        const int64_t s = row0 + i < p.n ? s_ld : -1;
        slot[i] = (int64_t)((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(s >> 32)) << 32 |
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)s));
        {
            typedef uint32_t u4 __attribute__((ext_vector_type(4)));
            const u4 t = __builtin_nontemporal_load(
                reinterpret_cast<const u4*>(p.rows + r * p.row_stride + 8 * lane));
            in[i] = make_uint4(t[0], t[1], t[2], t[3]);
        }
    }
#pragma unroll
    for (int i = 0; i < kStoreRowsPerWave; ++i)
        if (slot[i] >= 0 && slot[i] < p.num_slots) store_row(p, lane, slot[i], in[i]);
}

hipError_t launch_quantize_store(const StoreParams& p, hipStream_t stream) {
    const int64_t grid = (p.n + kStoreRows - 1) / kStoreRows;
    hipLaunchKernelGGL(quantize_store_kernel, dim3((unsigned)grid), dim3(kStoreThreads), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace dsv4
