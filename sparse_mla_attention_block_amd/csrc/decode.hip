// Sparse FP8 MLA decode kernels for gfx950 (CDNA4): the partial (split-K)
// kernel and the log-sum-exp combine kernel.
//
// Method sources (page titles):
//   vLLM PR #52212, gfx950 DSV4 sparse decode page, implementation item 1:
//     one 512-wide QK dot over 448 NoPE + 64 RoPE dims, 32-row guarded tiles,
//     masked tail, attention sink and invalid indices; item 2: split-K with
//     per-row active splits.
//   SGLang PR #26208 report, key source snippets: fp8_ds_mla row and page
//     layout, -1 invalid marker, top-k length mask; review highlights: a
//     masked or -inf score contributes exactly zero to the running sum.
//
// One workgroup = 8 waves serves one (token b, split s, head group g) and
// walks its slice of the token's entry list in tiles of 32 cache rows.
//   * Resolution (index -> page via the block table -> byte offsets) of 16
//     tiles at a time, one entry per lane, into an LDS ring; the next half
//     is resolved in steps spread over two tile periods so its dependent
//     loads overlap compute.
//   * Waves 4..7 ("producers", 8 lanes per cache row) keep the raw bytes of
//     the next two tiles in flight in registers, dequantise FP8 x 2^(code-127)
//     to bf16 and store
//     tile t+1 row-major into one half of a double-buffered LDS K tile while
//   * waves 0..3 ("consumers", one per 16-head MFMA row tile) run QK of tile
//     t on bf16 MFMA 16x16x32 (q held in registers) fused with the online
//     softmax (DPP row reductions, lazy rescaling: the running max only moves
//     when a score exceeds it by more than 2^8), writing bf16 probabilities;
//   * then all 8 waves run PV on bf16 MFMA, wave w owning output dims
//     [64w, 64w+64); the V operand comes straight from the row-major K tile
//     through the gfx950 LDS transpose read, so no transposed copy is kept.
// Rows that do not take part are stored as zeros, so a NaN in the cache can
// never reach an MFMA.  The running sum takes the fp32 probabilities, the PV
// operand their bf16 rounding.  With one split the epilogue folds the sink in
// and writes bf16 output and lse; with several it writes the split's
// normalised fp32 partial and lse.  Both leave through LDS as 16-byte stores.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "internal.hpp"

namespace dsv4 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;   // log2 units a score may exceed the running max by
constexpr int kHalfTiles = kMetaTiles / 2;

// 2^(code-127) as an fp32 value: UE8M0 code 0 is the subnormal 2^-127 and
// code 255 is NaN (the E8M0 encoding).
__device__ __forceinline__ float ue8m0_to_float(uint32_t code) {
    const uint32_t bits = code == 0u ? 0x00400000u : (code == 255u ? 0x7FC00000u : code << 23);
    return __uint_as_float(bits);
}

// 8 E4M3FN bytes times a power-of-two scale, as 8 bf16.  The gfx950 convert
// decodes OCP E4M3FN exactly to fp32; the product is exact and so is its
// bf16 rounding for every value a 4-bit-significand FP8 times 2^k can take
// inside bf16's normal range.
__device__ __forceinline__ bf16x8 dequant8(uint2 raw, float scale) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(raw.x, false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(raw.x, true);
    const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(raw.y, false);
    const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(raw.y, true);
    bf16x8 v;
    v[0] = (__bf16)(a[0] * scale);
    v[1] = (__bf16)(a[1] * scale);
    v[2] = (__bf16)(b[0] * scale);
    v[3] = (__bf16)(b[1] * scale);
    v[4] = (__bf16)(c[0] * scale);
    v[5] = (__bf16)(c[1] * scale);
    v[6] = (__bf16)(d[0] * scale);
    v[7] = (__bf16)(d[1] * scale);
    return v;
}

// Reductions over the 16 lanes of a DPP row (lanes sharing lane >> 4):
// quad xor 1, quad xor 2, half-row mirror, row mirror.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    return fmaxf(v, dpp<0x140>(v));
}
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    return v + dpp<0x140>(v);
}

// LDS transpose read (ds_read_b64_tr_b16): within each 16-lane group, lane i
// receives element i%4 of the 4-element vectors addressed by lanes i/4 + 4k,
// k = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const __bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
}

// Producer lane pl (0..255) owns row pl/8 of a tile and, of the row's 72
// eight-byte chunks (576 data bytes), chunks l8 + 8j for j = 0..8, l8 = pl%8:
// j < 7 are NoPE chunks (8 FP8 dims scaled by code j of the row's scale
// word), j = 7, 8 are RoPE chunks (4 bf16 dims each).  Every lane therefore
// runs the same instructions; a wave reads 64 contiguous bytes from each of
// 8 rows per load.  The raw chunks of a tile live in rr[O .. O+17] and the
// row's scale word in rr[O+18 .. O+19].  The loads are unconditional (a row
// that takes no part reads the pool's first row and is zeroed when stored),
// so they issue back to back.
// meta row: [byte offset of the row's data (-1 = the row takes no part),
//            byte offset of its scale word].
constexpr int kChunks = 9;

template <int O>
__device__ __forceinline__ void load_patch(const DecodeParams& p, const int64_t* meta, int prow,
                                           int l8, uint32_t (&rr)[64]) {
    const int64_t d = max(meta[2 * prow], (int64_t)0);
    const uint8_t* src = p.kv + d + 8 * l8;
    const uint2 sw = *reinterpret_cast<const uint2*>(p.kv + meta[2 * prow + 1]);
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
        const uint2 v = *reinterpret_cast<const uint2*>(src + 64 * j);
        rr[O + 2 * j] = v.x;
        rr[O + 2 * j + 1] = v.y;
    }
    rr[O + 18] = sw.x;
    rr[O + 19] = sw.y;
}

// Dequantises the chunks into the row-major K tile.
template <int O>
__device__ __forceinline__ void store_patch(const uint32_t (&rr)[64], const int64_t* meta, int prow,
                                            int l8, __bf16* Kn) {
    const bool ok = meta[2 * prow] >= 0;
    const uint64_t sw = ok ? ((uint64_t)rr[O + 19] << 32 | rr[O + 18]) : 0x7F7F7F7F7F7F7F7Full;
    __bf16* row = Kn + prow * kKnLd;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
        const uint2 raw = ok ? make_uint2(rr[O + 2 * j], rr[O + 2 * j + 1]) : make_uint2(0u, 0u);
        const float sc = ue8m0_to_float((uint32_t)(sw >> (8 * j)) & 0xFFu);
        *reinterpret_cast<bf16x8*>(row + 64 * j + 8 * l8) = dequant8(raw, sc);
    }
#pragma unroll
    for (int j = 7; j < kChunks; ++j) {
        const uint2 raw = ok ? make_uint2(rr[O + 2 * j], rr[O + 2 * j + 1]) : make_uint2(0u, 0u);
        *reinterpret_cast<uint2*>(row + kDNope + 32 * (j - 7) + 4 * l8) = raw;
    }
}

// Entry resolution helpers: effective position -> index -> page -> scale word.
__device__ __forceinline__ int32_t load_index(const DecodeParams& p, int b, int vl, int hi,
                                              int pos) {
    if (pos >= hi) return -1;
    const int col = pos < vl ? pos : p.topk + (pos - vl);
    return p.idx[(int64_t)b * p.idx_stride + col];
}

__device__ __forceinline__ int64_t lookup_page(const DecodeParams& p, int b, int32_t idx) {
    if (idx < 0) return -1;
    const int64_t blk = idx / p.bs;
    if (p.bt) {
        if (blk >= p.max_blocks) return -1;
        const int32_t pg = p.bt[(int64_t)b * p.bt_stride + blk];
        return (pg >= 0 && pg < p.num_blocks) ? pg : -1;
    }
    return blk < p.num_blocks ? blk : -1;
}

// Data and scale-word byte offsets of the row at (page, idx % bs); a row that
// takes no part gets data offset -1 and scale offset 0 (the pool's first
// bytes, read and discarded).
__device__ __forceinline__ void write_meta(const DecodeParams& p, int64_t* row, int64_t page,
                                           int32_t idx) {
    const int64_t off = idx % p.bs;
    row[0] = page >= 0 ? page * p.page_stride + off * kRowData : -1;
    row[1] = page >= 0 ? page * p.page_stride + (int64_t)p.bs * kRowData + off * kRowScale : 0;
}

// Reductions across the four 16-lane rows of a wave.  v_permlane16_swap
// exchanges the odd 16-lane rows of its first operand with the even rows of
// its second, v_permlane32_swap the upper 32 lanes of the first with the
// lower 32 of the second; with both operands holding v, every lane ends up
// with the two values of its row pair (half pair).  Written as inline asm:
// the optimiser of this compiler folds the builtins' second result into the
// first.  The s_nop covers the VALU-write to permlane-read hazard.
template <class Op>
__device__ __forceinline__ float xrow4(float v, Op op) {
    uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
    x = __builtin_bit_cast(uint32_t, op(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y)));
    y = x;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
    return op(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
}
__device__ __forceinline__ float xrow_max4(float v) {
    return xrow4(v, [](float p, float q) { return fmaxf(p, q); });
}
__device__ __forceinline__ float xrow_sum4(float v) {
    return xrow4(v, [](float p, float q) { return p + q; });
}

template <int HG>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(const DecodeParams p) {
    constexpr int MT = HG / 16;              // 16-head MFMA tiles; consumer wave w owns tile w
    static_assert(HG % 16 == 0 && HG <= kMaxHeadsPerGroup, "head group");
    using L = Smem<HG>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[L::bytes];
    __bf16* Kn = reinterpret_cast<__bf16*>(smem + L::kn);          // [2][32][520]
    __bf16* Pb = reinterpret_cast<__bf16*>(smem + L::pb);          // [HG][40]
    float* alpha_s = reinterpret_cast<float*>(smem + L::alpha);
    float* fin = reinterpret_cast<float*>(smem + L::fin);
    int* flags = reinterpret_cast<int*>(smem + L::flags);
    uint32_t* vmask = reinterpret_cast<uint32_t*>(smem + L::vmask);  // [32 tiles]
    int64_t* meta = reinterpret_cast<int64_t*>(smem + L::meta);    // [32 tiles][32][2]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;

    // Work unit.  Workgroups are handed to the 8 XCDs round-robin; the head
    // groups of one (token, split) are kXcds apart so they land on the same
    // XCD and share its L2 for the rows they both read.
    const int64_t Lb = blockIdx.x;
    const int x = (int)(Lb % kXcds);
    const int64_t r8 = Lb / kXcds;
    const int g = (int)(r8 % p.G);
    const int64_t unit = (r8 / p.G) * kXcds + x;
    if (unit >= p.units) return;
    const int b = (int)(unit / p.S);
    const int s = (int)(unit % p.S);
    const int h0 = g * HG;

    // This split's slice of the effective list main[0:vl] ++ swa, in chunks
    // rounded up to whole tiles.
    const int vl = p.valid_len ? min(max(p.valid_len[b], 0), p.topk) : p.topk;
    const int eff = vl + p.swa;
    int chunk = (eff + p.S - 1) / p.S;
    chunk = (chunk + kTile - 1) / kTile * kTile;
    const int lo = min(s * chunk, eff);
    const int hi = min(lo + chunk, eff);
    const int ntiles = (hi - lo + kTile - 1) / kTile;

    const bool consumer = wave < MT;
    const bool producer = wave >= 4;
    const int ptid = tid - 4 * 64;
    const int prow = ptid >> 3, l8 = ptid & 7;   // producer: tile row, chunk lane
    const int hc = 16 * wave + l16;              // consumer lane's head (within the group)
    auto meta_tile = [&](int t) { return meta + (t % kMetaTiles) * kTile * 2; };

    // One 64-register array per lane, used by role: consumers keep the q
    // row of their head in it (lane (l16, lg) holds dims 32*ks + 8*lg .. +7
    // of head 16*wave + l16 in rr[4ks..4ks+3], the B operand of QK);
    // producers keep two tiles of raw bytes in it (rr[0..19], rr[32..51]).
    uint32_t rr[64];
    float sink_l2 = -INFINITY;                   // consumer lane's sink, base-2 units
    if (consumer) {
        const u32x4* qp = reinterpret_cast<const u32x4*>(
            p.q + ((int64_t)b * p.H + h0 + hc) * kD + 8 * lg);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const u32x4 v = qp[4 * ks];
            rr[4 * ks] = v[0];
            rr[4 * ks + 1] = v[1];
            rr[4 * ks + 2] = v[2];
            rr[4 * ks + 3] = v[3];
        }
        if (p.sink) sink_l2 = p.sink[h0 + hc] * kLog2e;
    }

    // Resolution of 16 tiles: one entry per lane, then a per-tile bit mask of
    // the rows that take part (each wave covers two tiles).
    auto publish = [&](int first_tile, int64_t page, int32_t idx) {
        write_meta(p, meta_tile(first_tile) + 2 * tid, page, idx);
        const uint64_t bits = __builtin_amdgcn_ballot_w64(page >= 0);
        if (lane == 0) {
            vmask[(first_tile + 2 * wave) % kMetaTiles] = (uint32_t)bits;
            vmask[(first_tile + 2 * wave + 1) % kMetaTiles] = (uint32_t)(bits >> 32);
        }
    };
    {
        const int32_t idx = load_index(p, b, vl, hi, lo + tid);
        publish(0, lookup_page(p, b, idx), idx);
    }
    __syncthreads();

    if (producer) {
        if (ntiles > 0) load_patch<0>(p, meta_tile(0), prow, l8, rr);
        if (ntiles > 1) load_patch<32>(p, meta_tile(1), prow, l8, rr);
        if (ntiles > 0) store_patch<0>(rr, meta_tile(0), prow, l8, Kn);
        if (ntiles > 2) load_patch<0>(p, meta_tile(2), prow, l8, rr);
    }
    __syncthreads();

    // Online-softmax state of a consumer lane's head, in base-2 units
    // (replicated over the lane's four 16-lane rows).
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Staged resolution of the next half (16 tiles), one entry per lane.
    int32_t r_idx = -1;
    int64_t r_pg = -1;

    // One tile period; rr[O..O+19] holds tile t+1's raw bytes and receives
    // tile t+3's (O = 32 for even t, 0 for odd t).
    auto step = [&](int t, auto off) __attribute__((always_inline)) {
        constexpr int O = decltype(off)::value;
        const int ph = t % kHalfTiles;
        const bool resolving = t - ph + kHalfTiles < ntiles;   // a next half exists
        const int half_base = lo + (t - ph + kHalfTiles) * kTile;
        // ---- B: QK + softmax (consumers) | dequant t+1, load t+3 (producers)
        if (resolving && ph == 0) r_idx = load_index(p, b, vl, hi, half_base + tid);
        if (consumer) {
            // S^T = K q^T: A operand = K rows (entries), B operand = q (heads).
            const __bf16* K = Kn + (t & 1) * kTile * kKnLd;
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
            const __bf16* k0 = &K[l16 * kKnLd + 8 * lg];
            const __bf16* k1 = &K[(16 + l16) * kKnLd + 8 * lg];
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
                const bf16x8 kb0 = *reinterpret_cast<const bf16x8*>(k0 + 32 * ks);
                const bf16x8 kb1 = *reinterpret_cast<const bf16x8*>(k1 + 32 * ks);
                const bf16x8 qb = __builtin_bit_cast(
                    bf16x8, u32x4{rr[4 * ks], rr[4 * ks + 1], rr[4 * ks + 2], rr[4 * ks + 3]});
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb0, qb, s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb1, qb, s1, 0, 0, 0);
            }
            // lane holds the scores of head hc for rows 4lg + r (s0) and 16 + 4lg + r (s1).
            const uint32_t vm = vmask[t % kMetaTiles];
            float x[8];
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[r] = (vm >> (4 * lg + r)) & 1u ? s0[r] * p.qk_scale_log2 : -INFINITY;
                x[4 + r] = (vm >> (16 + 4 * lg + r)) & 1u ? s1[r] * p.qk_scale_log2 : -INFINITY;
                mx = fmaxf(mx, fmaxf(x[r], x[4 + r]));
            }
            mx = xrow_max4(mx);
            // Move the running max only when a score exceeds it by more than
            // the slack (always on the first valid score).
            const bool move = mx > m_run + kRescaleSlack;
            const float m_use = move ? mx : m_run;
            const float a = move ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;   // 0 if m_run = -inf
            float e[8], psum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                e[i] = x[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[i] - m_use);
                psum += e[i];
            }
            l_run = l_run * a + xrow_sum4(psum);
            m_run = m_use;
            bf16x8 pv;
#pragma unroll
            for (int i = 0; i < 8; ++i) pv[i] = (__bf16)e[i];
            __bf16* prow_p = Pb + hc * kPLd + 4 * lg;
            *reinterpret_cast<uint2*>(prow_p) = __builtin_bit_cast(
                uint2, __builtin_shufflevector(pv, pv, 0, 1, 2, 3));
            *reinterpret_cast<uint2*>(prow_p + 16) = __builtin_bit_cast(
                uint2, __builtin_shufflevector(pv, pv, 4, 5, 6, 7));
            if (lg == 0) alpha_s[hc] = a;
            const bool any = __builtin_amdgcn_ballot_w64(move) != 0;
            if (lane == 0) flags[wave] = any ? 1 : 0;
        }
        if (producer) {
            if (t + 1 < ntiles)
                store_patch<O>(rr, meta_tile(t + 1), prow, l8, Kn + ((t + 1) & 1) * kTile * kKnLd);
            if (t + 3 < ntiles) load_patch<O>(p, meta_tile(t + 3), prow, l8, rr);
        }
        __syncthreads();

        // ---- C: PV (all waves) into output dims [64w, 64w+64).
        if (resolving && ph == 0) r_pg = lookup_page(p, b, r_idx);
        if (resolving && ph == 1) publish(t - ph + kHalfTiles, r_pg, r_idx);
        {
            const __bf16* K = Kn + (t & 1) * kTile * kKnLd;
            bool rescale = false;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) rescale |= flags[mt] != 0;
            bf16x8 pa[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                pa[mt] = *reinterpret_cast<const bf16x8*>(&Pb[(16 * mt + l16) * kPLd + 8 * lg]);
                if (rescale) {
                    const f32x4 al = *reinterpret_cast<const f32x4*>(&alpha_s[16 * mt + 4 * lg]);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] *= al;
                }
            }
            // V operand: lane j of 16-lane group lg points at rows 8lg + 4h + j/4,
            // dims dimb + 4(j%4); the transpose read hands lane i dim dimb + i of
            // rows 8lg + 4h .. +3.
            const __bf16* vrow = &K[(8 * lg + (l16 >> 2)) * kKnLd + 64 * wave + 4 * (l16 & 3)];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const i16x4 v0 = lds_read_tr16(vrow + 16 * nt);
                const i16x4 v1 = lds_read_tr16(vrow + 4 * kKnLd + 16 * nt);
                const bf16x8 vb = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[mt], vb, acc[mt][nt],
                                                                          0, 0, 0);
            }
        }
        __syncthreads();
    };

    for (int t = 0; t < ntiles; t += 2) {
        step(t, std::integral_constant<int, 32>{});
        if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 0>{});
    }

    // Epilogue: output scale and lse of each head (consumer lanes of row 0,
    // one head each).
    const bool direct = p.S == 1;
    if (consumer && lg == 0) {
        const int h = h0 + hc;
        float scale, lse;
        if (direct && p.sink) {
            const float M = fmaxf(m_run, sink_l2);
            const float em = __builtin_amdgcn_exp2f(m_run - M);
            const float D = l_run * em + __builtin_amdgcn_exp2f(sink_l2 - M);
            scale = em * __builtin_amdgcn_rcpf(D);
            lse = (M + __builtin_amdgcn_logf(D)) * kLn2;
        } else if (l_run > 0.f) {
            scale = __builtin_amdgcn_rcpf(l_run);
            lse = (m_run + __builtin_amdgcn_logf(l_run)) * kLn2;
        } else {
            scale = 0.f;
            lse = -INFINITY;
        }
        fin[hc] = scale;
        if (direct) {
            if (p.lse) p.lse[(int64_t)b * p.H + h] = lse;
        } else {
            p.part_lse[((int64_t)b * p.H + h) * p.S + s] = lse;
        }
    }
    __syncthreads();

    // Output through LDS as bf16 (the final output, or the split's partial):
    // lane holds O[16mt + 4lg + r][64w + 16nt + l16].
    constexpr int LD = L::stage_ld;
    __bf16* st = reinterpret_cast<__bf16*>(smem + L::stage);        // [HG][520]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const f32x4 sc = *reinterpret_cast<const f32x4*>(&fin[16 * mt + 4 * lg]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                st[(16 * mt + 4 * lg + r) * LD + 64 * wave + 16 * nt + l16] =
                    (__bf16)(acc[mt][nt][r] * sc[r]);
    }
    __syncthreads();
    uint16_t* dst;
    int64_t row_stride;
    if (direct) {
        dst = p.out + ((int64_t)b * p.H + h0) * kD;
        row_stride = kD;
    } else {
        dst = p.part_o + (((int64_t)b * p.H + h0) * p.S + s) * kD;
        row_stride = (int64_t)p.S * kD;
    }
    for (int c = tid; c < HG * (kD / 8); c += kThreads) {
        const int row = c >> 6, col = (c & 63) * 8;
        *reinterpret_cast<bf16x8*>(dst + row * row_stride + col) =
            *reinterpret_cast<const bf16x8*>(&st[row * LD + col]);
    }
}

// Merge of split partials with the sink; one workgroup per (token, head),
// 4 output dims per lane.  Splits are taken NB at a time (NB = the split
// count rounded up to a power of two, at most 32): every partial and lse load
// of a batch is issued before any is used (one memory round trip per batch),
// and batches are merged with an online rescale.
template <int kCombineBatch>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const CombineParams p) {
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % p.H);
    const float* ls = p.part_lse + bh * p.S;
    const uint16_t* po = p.part_o + bh * p.S * kD + threadIdx.x * 4;
    float M = p.sink ? p.sink[h] : -INFINITY;
    float D = p.sink ? 1.f : 0.f;                    // e^{sink - M} with M = sink
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < p.S; s0 += kCombineBatch) {
        const int n = min(kCombineBatch, p.S - s0);
        uint2 v[kCombineBatch];
        float l[kCombineBatch];
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) {
            l[j] = j < n ? ls[s0 + j] : -INFINITY;
            v[j] = j < n ? *reinterpret_cast<const uint2*>(po + (int64_t)(s0 + j) * kD)
                         : make_uint2(0u, 0u);
        }
        float cm = -INFINITY;
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) cm = fmaxf(cm, l[j]);
        const float M2 = fmaxf(M, cm);
        if (M2 == -INFINITY) continue;               // nothing so far
        const float c = __builtin_amdgcn_exp2f((M - M2) * kLog2e);   // 0 when M = -inf
        D *= c;
        o *= c;
#pragma unroll
        for (int j = 0; j < kCombineBatch; ++j) {
            const float w = l[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((l[j] - M2) * kLog2e);
            D += w;
            const f32x4 pv = {__uint_as_float(v[j].x << 16), __uint_as_float(v[j].x & 0xFFFF0000u),
                              __uint_as_float(v[j].y << 16), __uint_as_float(v[j].y & 0xFFFF0000u)};
            o += w * pv;
        }
        M = M2;
    }
    float lse = -INFINITY;
    if (M != -INFINITY) {
        o *= 1.f / D;
        lse = M + __builtin_amdgcn_logf(D) * kLn2;
    }
    uint2 packed;
    packed.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[0]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[1]) << 16);
    packed.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[2]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[3]) << 16);
    *reinterpret_cast<uint2*>(p.out + bh * kD + threadIdx.x * 4) = packed;
    if (threadIdx.x == 0 && p.lse) p.lse[bh] = lse;
}

hipError_t launch_decode_partial(const DecodeParams& p, int heads_per_group, int64_t grid,
                                 hipStream_t stream) {
    const dim3 g((unsigned)grid), blk(kThreads);
    switch (heads_per_group) {
        case 16: hipLaunchKernelGGL(decode_partial_kernel<16>, g, blk, 0, stream, p); break;
        case 32: hipLaunchKernelGGL(decode_partial_kernel<32>, g, blk, 0, stream, p); break;
        case 48: hipLaunchKernelGGL(decode_partial_kernel<48>, g, blk, 0, stream, p); break;
        case 64: hipLaunchKernelGGL(decode_partial_kernel<64>, g, blk, 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
    const dim3 g((unsigned)((int64_t)p.B * p.H)), blk(kCombineThreads);
    if (p.S <= 4)
        hipLaunchKernelGGL(combine_kernel<4>, g, blk, 0, stream, p);
    else if (p.S <= 8)
        hipLaunchKernelGGL(combine_kernel<8>, g, blk, 0, stream, p);
    else if (p.S <= 16)
        hipLaunchKernelGGL(combine_kernel<16>, g, blk, 0, stream, p);
    else
        hipLaunchKernelGGL(combine_kernel<32>, g, blk, 0, stream, p);
    return hipGetLastError();
}

}  // namespace dsv4
