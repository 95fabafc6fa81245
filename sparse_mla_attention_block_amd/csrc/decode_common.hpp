// Device helpers shared by the decode kernels (the pipelined partial kernel,
// the short-split kernel, the two-kernel path and the gather floor): vector
// types, the FP8 row decoder, the LDS K-tile layout, row loads and stores,
// entry resolution, and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "device_util.hpp"
#include "internal.hpp"

namespace dsv4 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int64_t i64x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;   // log2 units a score may exceed the running max by
constexpr int kHalfTiles = kMetaTiles / 2;

// Two FP8 E4M3FN bytes of `packed` (bytes 0-1, or 2-3 with HI) times a power
// of two, as two bf16, in one gfx950 scaled convert.  The instruction takes
// only the exponent field of its fp32 scale operand, so UE8M0 code c is
// passed as the float bits c << 23: code 0 is 2^-127 and 255 is NaN, the
// E8M0 meanings.  For every FP8 byte and scale codes from 0 to 255 the
// result equals the bf16 rounding of the exact product (checked on gfx950
// against an exact decoder).  Inline asm: the compiler's builtin for this
// instruction returns the low byte's value in both halves.
template <bool HI>
__device__ __forceinline__ uint32_t cvt_scaled_pk(uint32_t packed, float scale) {
    uint32_t r;
    if (HI)
        asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, %2 op_sel:[1,0,0]" : "=v"(r) : "v"(packed), "v"(scale));
    else
        asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, %2" : "=v"(r) : "v"(packed), "v"(scale));
    return r;
}

// 8 E4M3FN bytes times 2^(code-127), as 8 bf16.
__device__ __forceinline__ bf16x8 dequant8(uint2 raw, uint32_t code) {
    const float scale = __uint_as_float(code << 23);
    return __builtin_bit_cast(bf16x8, u32x4{cvt_scaled_pk<false>(raw.x, scale),
                                            cvt_scaled_pk<true>(raw.x, scale),
                                            cvt_scaled_pk<false>(raw.y, scale),
                                            cvt_scaled_pk<true>(raw.y, scale)});
}

// Source of rows that take no part and of tiles past the end of a split: 576
// zero data bytes and a zero scale word, which dequantise to exact zeros, or
// a whole zero bf16 row (1024 bytes) for dense sources, so a NaN anywhere in
// the cache can never reach an MFMA.
constexpr int kDenseRow = kD * 2;
__device__ __attribute__((aligned(64))) const uint8_t kZeroRow[kDenseRow] = {};

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

// K tile layout: row-major, 512 bf16 (1024 B) per row, the row's 64
// sixteen-byte units permuted by XOR with swz(row) (bits of the row number
// moved to unit bits 3, 1-2 and 4).  The permutation was chosen by measuring
// the LDS bank-conflict counter for the kernel's four access patterns on
// gfx950: the QK fragment reads (16 rows, one unit each, per 16 lanes), the
// PV transpose reads (4 rows x four 8-byte pieces per 16 lanes), and the
// producers' 16-byte and 8-byte stores (rows r and r+4 per 16 lanes).
__device__ __forceinline__ int swz(int row) {
    return 8 * (row & 1) + 2 * ((row >> 1) & 3) + 16 * ((row >> 3) & 1);
}

// Element offset of element `elem` of row `row` in a K tile.
__device__ __forceinline__ int kofs(int row, int elem) {
    return row * kD + ((((elem >> 3) ^ swz(row))) << 3) + (elem & 7);
}

// Producer lane l of producer wave v owns row 8v + l/16 + 4((l/8)%2) of a
// tile (so 16 lanes store rows r and r+4) and, of the row's 72 eight-byte
// chunks (576 data bytes), chunks l8 + 8j for j = 0..8, l8 = l%8: j < 7 are
// NoPE chunks (8 FP8 dims scaled by code j of the row's scale word), j = 7, 8
// are RoPE chunks (4 bf16 dims each).  Every lane therefore runs the same
// instructions; a wave reads 64 contiguous bytes from each of 8 rows per
// load.  The raw chunks of a tile live in rr[O .. O+17] and the row's scale
// word in rr[O+18 .. O+19].  The loads are unconditional: a row that takes no
// part, or a tile past the end of the split, reads the zero row.  With no
// branch around them the compiler can count the loads in flight and wait for
// one tile's loads while the next tile's are still outstanding.
// meta row: [address of the row's 576 data bytes, address of its scale word]
// (the zero row for a row that takes no part).
constexpr int kChunks = 9;

// Global-memory pointers (address space 1), so the loads are global loads
// (counted by vmcnt alone) rather than flat ones.
typedef const __attribute__((address_space(1))) uint8_t gbyte;
typedef const __attribute__((address_space(1))) uint64_t gu64;

struct PatchSrc {
    gbyte* data;
    gbyte* scale;
};

// A producer lane's row addresses, read as one 16-byte LDS word (the slot
// always exists; a dead tile's stale entry is replaced after the read).
__device__ __forceinline__ PatchSrc patch_src(const int64_t* meta, int prow, bool live) {
    const i64x2 m = *reinterpret_cast<const i64x2*>(meta + 2 * prow);
    const int64_t z = reinterpret_cast<int64_t>(kZeroRow);
    return PatchSrc{(gbyte*)(live ? m[0] : z), (gbyte*)(live ? m[1] : z + kRowData)};
}

template <int O>
__device__ __forceinline__ void load_patch(PatchSrc a, int l8, uint32_t (&rr)[64]) {
    gbyte* src = a.data + 8 * l8;
    const uint64_t sw = *(gu64*)a.scale;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
        const uint64_t v = *(gu64*)(src + 64 * j);
        rr[O + 2 * j] = (uint32_t)v;
        rr[O + 2 * j + 1] = (uint32_t)(v >> 32);
    }
    rr[O + 18] = (uint32_t)sw;
    rr[O + 19] = (uint32_t)(sw >> 32);
}

// Dequantises the chunks into the K tile.  With SCRUB every element that is
// not finite after dequantisation (an FP8 NaN byte, a NaN scale code, a
// product past the bf16 range, a NaN or infinite RoPE value) is stored as 0.
template <int O, bool SCRUB>
__device__ __forceinline__ void store_patch(const uint32_t (&rr)[64], int prow, int l8,
                                            __bf16* Kt) {
    const uint64_t sw = (uint64_t)rr[O + 19] << 32 | rr[O + 18];
#pragma unroll
    for (int j = 0; j < 7; ++j) {
        const uint2 raw = make_uint2(rr[O + 2 * j], rr[O + 2 * j + 1]);
        bf16x8 v = dequant8(raw, (uint32_t)(sw >> (8 * j)) & 0xFFu);
        if (SCRUB) {
            u32x4 w = __builtin_bit_cast(u32x4, v);
            w = u32x4{scrub_pair(w[0]), scrub_pair(w[1]), scrub_pair(w[2]), scrub_pair(w[3])};
            v = __builtin_bit_cast(bf16x8, w);
        }
        *reinterpret_cast<bf16x8*>(Kt + kofs(prow, 64 * j + 8 * l8)) = v;
    }
#pragma unroll
    for (int j = 7; j < kChunks; ++j) {
        uint2 raw = make_uint2(rr[O + 2 * j], rr[O + 2 * j + 1]);
        if (SCRUB) raw = make_uint2(scrub_pair(raw.x), scrub_pair(raw.y));
        *reinterpret_cast<uint2*>(Kt + kofs(prow, kDNope + 32 * (j - 7) + 4 * l8)) = raw;
    }
}

// Dense bf16 source (the two-kernel path's gathered rows): lane l8 of a row
// holds its 16-byte units 8j + l8, j = 0..7 (32 registers per tile), stored
// into the K tile exactly where the FP8 path stores its dequantised units.
typedef const __attribute__((address_space(1))) u32x4 gu32x4;

__device__ __forceinline__ gbyte* dense_src(const int64_t* meta, int prow, bool live) {
    const int64_t m = meta[2 * prow];
    return (gbyte*)(live ? m : reinterpret_cast<int64_t>(kZeroRow));
}

template <int O>
__device__ __forceinline__ void load_dense(gbyte* src, int l8, uint32_t (&rr)[64]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const u32x4 v = *(gu32x4*)(src + 128 * j + 16 * l8);
        rr[O + 4 * j] = v[0];
        rr[O + 4 * j + 1] = v[1];
        rr[O + 4 * j + 2] = v[2];
        rr[O + 4 * j + 3] = v[3];
    }
}

template <int O>
__device__ __forceinline__ void store_dense(const uint32_t (&rr)[64], int prow, int l8,
                                            __bf16* Kt) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
        *reinterpret_cast<u32x4*>(Kt + kofs(prow, 64 * j + 8 * l8)) =
            u32x4{rr[O + 4 * j], rr[O + 4 * j + 1], rr[O + 4 * j + 2], rr[O + 4 * j + 3]};
}

// A dense entry: row `pos` of token b's gathered rows takes part when it
// lies in [lo, hi) and its mask byte is 0.  The mask load is unconditional
// (an out-of-range position reads the split's first entry).
__device__ __forceinline__ bool dense_live(const DecodeParams& p, int b, int lo, int hi, int pos) {
    const int col = pos < hi ? pos : lo;
    const uint8_t m = p.mask[(int64_t)b * p.idx_stride + col];
    return pos < hi && m == 0;
}

__device__ __forceinline__ void write_dense_meta(const DecodeParams& p, int64_t* row, int b,
                                                 int pos, bool live) {
    const uint8_t* r = p.kv + ((int64_t)b * p.idx_stride + pos) * kDenseRow;
    row[0] = reinterpret_cast<int64_t>(live ? r : kZeroRow);
    row[1] = 0;
}

// Entry resolution helpers: effective position -> index -> page.  Both loads
// are unconditional (an out-of-range position reads column 0, a masked index
// block 0 of the row's table) and the result is selected afterwards, so the
// loop they sit in has no branch around a load.
__device__ __forceinline__ int32_t load_index(const DecodeParams& p, int b, int vl, int hi,
                                              int pos) {
    const bool in = pos < hi;
    const int col = in ? (pos < vl ? pos : p.topk + (pos - vl)) : 0;
    const int32_t v = p.idx[(int64_t)b * p.idx_stride + col];
    return in ? v : -1;
}

// The pool an entry resolves in: the second (SWA) pool of a dual cache for
// entries of the SWA part (effective position >= vl), else the first.  Both
// pools have a block table or neither does, so the table test stays uniform.
struct Pool {
    const uint8_t* kv;
    const int32_t* bt;
    int64_t num_blocks, bt_stride, page_stride;
    int32_t bs, max_blocks;
};

__device__ __forceinline__ Pool pool_of(const DecodeParams& p, bool swa_entry) {
    const bool u = swa_entry && p.kv2 != nullptr;
    return Pool{u ? p.kv2 : p.kv,
                u ? p.bt2 : p.bt,
                u ? p.num_blocks2 : p.num_blocks,
                u ? p.bt_stride2 : p.bt_stride,
                u ? p.page_stride2 : p.page_stride,
                u ? p.bs2 : p.bs,
                u ? p.max_blocks2 : p.max_blocks};
}

__device__ __forceinline__ int64_t lookup_page(const DecodeParams& p, const Pool& pl, int seq,
                                               int32_t idx) {
    const bool ok = idx >= 0;
    const int64_t blk = (ok ? idx : 0) / pl.bs;
    if (p.bt) {
        const bool inb = ok && blk < pl.max_blocks;
        const int32_t pg = pl.bt[(int64_t)seq * pl.bt_stride + (inb ? blk : 0)];
        return (inb && pg >= 0 && pg < pl.num_blocks) ? pg : -1;
    }
    return (ok && blk < pl.num_blocks) ? blk : -1;
}

// lookup_page cut in two, for resolving several entries a thread with all
// their table loads in flight together: the table column to load (0 for an
// entry that takes no part), then the page from the loaded word (-1: takes
// no part; without a table the block number is the page).
__device__ __forceinline__ int64_t table_column(const Pool& pl, int32_t idx) {
    const int64_t blk = idx / pl.bs;
    return idx >= 0 && blk < pl.max_blocks ? blk : (int64_t)0;
}

__device__ __forceinline__ int64_t page_from_word(const DecodeParams& p, const Pool& pl,
                                                  int32_t idx, int32_t raw) {
    if (idx < 0) return -1;
    const int64_t blk = idx / pl.bs;
    if (p.bt) return blk < pl.max_blocks && raw >= 0 && raw < pl.num_blocks ? raw : -1;
    return blk < pl.num_blocks ? blk : -1;
}

// Data and scale-word addresses of the row at (page, idx % bs); the zero row
// for a row that takes no part.
__device__ __forceinline__ void write_meta(const Pool& pl, int64_t* row, int64_t page,
                                           int32_t idx) {
    const int64_t off = idx % pl.bs;
    const uint8_t* pg = pl.kv + page * pl.page_stride;
    row[0] = reinterpret_cast<int64_t>(page >= 0 ? pg + off * kRowData : kZeroRow);
    row[1] = reinterpret_cast<int64_t>(
        page >= 0 ? pg + (int64_t)pl.bs * kRowData + off * kRowScale : kZeroRow + kRowData);
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

// ---- Helpers of the short-split kernel ----

// K tile: 64 rows of 512 bf16 at a stride of 520 elements (1040 bytes).  The
// 16 rows one QK read spans then start 4 banks apart, and the element offset
// of (row, dim) is row * 520 + dim.
constexpr int kShortLd = kD + 8;

// Stand-in for a sink when there is none.
__device__ const float kZeroFloat = 0.f;

// A global-memory (address space 1) view of a pointer, so that a load
// through it is a global load, counted by vmcnt alone: a select between two
// pointers of different origins would otherwise make it a flat load, after
// which the compiler can only wait for all outstanding loads.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* global(const T* ptr) {
    return (const __attribute__((address_space(1))) T*)ptr;
}

// Resolution of entry `idx` (-1: no part) of sequence `seq` in two stages,
// so that the block-table loads of several entries are in flight together:
// the table word (TABLE: a load, unconditional), then the row addresses
// (the zero row when the entry takes no part; `live` tells which).  Without
// a table, idx is a pool slot.
template <bool TABLE>
__device__ __forceinline__ int32_t table_word(const DecodeParams& p, uint32_t seq, int32_t idx) {
    if constexpr (!TABLE) return 0;
    const uint32_t blk = fdiv(idx >= 0 ? (uint32_t)idx : 0u, p.fd_bs);
    const bool inb = idx >= 0 && blk < (uint32_t)p.max_blocks;
    return *global(p.bt + (int64_t)seq * p.bt_stride + (inb ? blk : 0u));
}

template <bool TABLE>
__device__ __forceinline__ PatchSrc row_source(const DecodeParams& p, int32_t idx, int32_t word,
                                               bool& live) {
    const uint32_t ui = idx >= 0 ? (uint32_t)idx : 0u;
    const uint32_t blk = fdiv(ui, p.fd_bs);
    const uint32_t off = ui - blk * p.fd_bs.d;
    int64_t page;
    if constexpr (TABLE) {
        const bool inb = idx >= 0 && blk < (uint32_t)p.max_blocks;
        page = (inb && word >= 0 && word < p.num_blocks) ? (int64_t)word : -1;
    } else {
        page = (idx >= 0 && blk < p.num_blocks) ? (int64_t)blk : -1;
    }
    live = page >= 0;
    const uint8_t* base = p.kv + (live ? page : 0) * p.page_stride;
    const int64_t z = reinterpret_cast<int64_t>(kZeroRow);
    const int64_t d = reinterpret_cast<int64_t>(base + off * kRowData);
    const int64_t s = reinterpret_cast<int64_t>(base + p.fd_bs.d * kRowData + off * kRowScale);
    return PatchSrc{(gbyte*)(live ? d : z), (gbyte*)(live ? s : z + kRowData)};
}

// Reductions over groups of N consecutive lanes (N = 8 or 16) of a DPP row.
template <int N>
__device__ __forceinline__ float group_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    if constexpr (N == 16) v = fmaxf(v, dpp<0x140>(v));
    return v;
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    if constexpr (N == 16) v += dpp<0x140>(v);
    return v;
}

// Position of entry e (0..63, a multiple of 4) of a super-tile in the MFMA
// k order of PV: within each 32-entry k-step, k = 8g + 4h + i holds entry
// 16h + 4g + i, the order in which the LDS transpose read delivers V.
__device__ __forceinline__ int k_slot(int e) {
    return (e & 32) + 8 * ((e >> 2) & 3) + 4 * ((e >> 4) & 1);
}

// Dequantised row chunks of one lane into the padded K tile.
template <int O, bool SCRUB>
__device__ __forceinline__ void store_row(const uint32_t (&rr)[64], int prow, int l8,
                                          __bf16* Kt) {
    const uint64_t sw = (uint64_t)rr[O + 19] << 32 | rr[O + 18];
    __bf16* dst = Kt + prow * kShortLd + 8 * l8;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
        bf16x8 v = dequant8(make_uint2(rr[O + 2 * j], rr[O + 2 * j + 1]),
                            (uint32_t)(sw >> (8 * j)) & 0xFFu);
        if (SCRUB) {
            u32x4 w = __builtin_bit_cast(u32x4, v);
            w = u32x4{scrub_pair(w[0]), scrub_pair(w[1]), scrub_pair(w[2]), scrub_pair(w[3])};
            v = __builtin_bit_cast(bf16x8, w);
        }
        *reinterpret_cast<bf16x8*>(dst + 64 * j) = v;
    }
    __bf16* rdst = Kt + prow * kShortLd + kDNope + 4 * l8;
#pragma unroll
    for (int j = 7; j < kChunks; ++j) {
        uint2 raw = make_uint2(rr[O + 2 * j], rr[O + 2 * j + 1]);
        if (SCRUB) raw = make_uint2(scrub_pair(raw.x), scrub_pair(raw.y));
        *reinterpret_cast<uint2*>(rdst + 32 * (j - 7)) = raw;
    }
}

}  // namespace dsv4
