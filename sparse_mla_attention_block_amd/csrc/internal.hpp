// Internal declarations shared by the host API and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fastdiv.hpp"

namespace dsv4 {

// Row geometry of the fp8_ds_mla cache (SGLang PR #26208 report, key source
// snippets: D_QK 512 = 448 NoPE + 64 RoPE, 576 data bytes and 8 scale bytes
// per token).
constexpr int kD = 512;
constexpr int kDNope = 448;
constexpr int kDRope = 64;
constexpr int kRowData = 576;
constexpr int kRowScale = 8;
constexpr int kRowBytes = kRowData + kRowScale;

// Decode kernel shape: 8 waves of 64 lanes, 32 cache rows per tile (the
// "BK32" tiles of the vLLM PR #52212 page), up to 64 heads per workgroup.
constexpr int kThreads = 512;
constexpr int kTile = 32;
constexpr int kMaxHeadsPerGroup = 64;
constexpr int kMaxSplits = 64;
constexpr int kMaxAutoSplits = 32;  // selector cap (the long-context low-batch cap of the vLLM PR #52212 page)
constexpr int kMaxSplitTiles = 8;   // selector: tiles per split before larger head groups win
constexpr int kCUs = 256;           // MI355X compute units
constexpr int kXcds = 8;            // accelerator dies; workgroups go round-robin
constexpr int kCombineThreads = 128;  // whole-row combine: 4 output dims per thread
constexpr int kGatherThreads = 256;   // two-kernel path gather: 32 entries x 8 lanes

// Short-split kernel: splits of at most kShortMaxSuper super-tiles of
// kShortRows cache rows, every phase on all 8 waves.
constexpr int kShortRows = 64;
constexpr int kShortMaxSuper = 2;
constexpr int kShortMaxEntries = kShortRows * kShortMaxSuper;

// LDS tile geometry.  K tiles are row-major [32][512] bf16 with the 16-byte
// units of each row permuted (see the kernel); probabilities [HG][40] bf16.
constexpr int kPLd = kTile + 8;
constexpr int kMetaTiles = 32;      // resolved-entry ring: two halves of 16 tiles

// LDS carve-up of the partial kernel (bytes).  K tiles rotate through three
// buffers (one being written, one read by QK, one read by PV); probabilities,
// rescale factors and rescale flags through two.
constexpr int kKBufs = 3;

template <int HG>
struct Smem {
    static constexpr int fin = 0;                                  // [HG] f32
    static constexpr int flags = fin + HG * 4;                     // [2][4] int
    static constexpr int alpha = flags + 32;                       // [2][HG] f32
    static constexpr int pb = alpha + 2 * HG * 4;                  // [2][HG][40] bf16
    static constexpr int pb_buf = HG * kPLd * 2;
    static constexpr int vmask = pb + 2 * pb_buf;                  // [32 tiles] u32
    static constexpr int kn = vmask + kMetaTiles * 4;              // [3][32][512] bf16
    static constexpr int kn_buf = kTile * kD * 2;
    static constexpr int meta = kn + kKBufs * kn_buf;              // [32 tiles][32][2] int64
    static constexpr int bytes = meta + kMetaTiles * kTile * 16;
    static_assert(pb % 16 == 0 && kn % 16 == 0 && meta % 16 == 0, "alignment");
    static_assert(bytes <= 160 * 1024, "LDS");
};

constexpr size_t lds_bytes_for(int hg) {
    return hg == 16 ? Smem<16>::bytes
         : hg == 32 ? Smem<32>::bytes
         : hg == 48 ? Smem<48>::bytes
                    : Smem<64>::bytes;
}

struct DecodeParams {
    const uint16_t* q;          // bf16 [B, H, 512]
    const uint8_t* kv;          // pages
    const int32_t* bt;          // [B / sq, bt_stride] or null
    const int32_t* idx;         // [B, idx_stride]
    const int32_t* valid_len;   // [B / sq] or null
    const uint8_t* mask;        // dense source only: [B, idx_stride], 1 = no part
    // Dual cache: the pool SWA entries resolve in (kv2 null: one pool).
    const uint8_t* kv2;
    const int32_t* bt2;
    int64_t num_blocks2, bt_stride2, page_stride2;
    int32_t bs2, max_blocks2;
    const float* sink;          // [H] or null
    uint16_t* out;              // bf16 [B, H, 512] (direct output, S == 1)
    float* lse;                 // [B, H] or null (direct output, S == 1)
    uint16_t* part_o;           // bf16 [B, H, S, 512] (S > 1)
    float* part_lse;            // [B, H, S] (S > 1)
    int64_t num_blocks;
    int64_t bt_stride;
    int64_t page_stride;
    int64_t idx_stride;
    int64_t units;              // work units: B * S, or B * bal with balanced splits
    int32_t B, H, topk, swa, bs, max_blocks, S, G;
    // Balanced splits (pipelined kernel): 0 = off; else the split budget per
    // token, with S the split slots per (token, head) row of the partials.
    int32_t bal;
    int32_t bal_hi;             // ceil(ceil((topk + swa) / bal) / 32): the uniform tiles per split
    int32_t sq;                 // query tokens per sequence (block-table row / valid_len entry)
    float qk_scale_log2;        // sm_scale * log2(e)
    // Launch-time divisors (the short-split kernel): splits, head groups,
    // tokens per sequence, and the block sizes of the two pools.
    FastDiv fd_S, fd_G, fd_sq, fd_bs, fd_bs2;
    // Measurement aid (short-split kernel only): per-workgroup phase stamps,
    // kTimelineStamps words per workgroup, or null.
    uint64_t* timeline;
    // Either partial kernel, with a block table and uniform splits (the
    // pipelined one with at most 1024 index columns a split): the req-local
    // -> global conversion of every index column, int32 [B, topk + swa],
    // fill -1; or null.
    int32_t* slots;
};

constexpr int kTimelineStamps = 10;

struct CombineParams {
    const uint16_t* part_o;     // bf16 [B, H, S, 512]
    const float* part_lse;
    const float* sink;
    uint16_t* out;
    float* lse;
    int32_t B, H, S;
};

struct ConvertParams {
    const int32_t* req_id;
    const int32_t* bt;
    const int32_t* ti;
    const int32_t* cu;
    int32_t* out;
    int64_t bt_stride;
    int64_t ti_stride;
    int32_t num_reqs, max_blocks, num_tokens, width, bs, fill;
    int32_t sq;                 // without req_id: token t reads table row t / sq
};

struct StoreParams {
    const uint16_t* rows;       // bf16 [n, row_stride]
    const int64_t* slots;       // [n] global slots
    uint8_t* kv;                // pages
    int64_t n;
    int64_t row_stride;         // elements
    int64_t num_blocks;
    int64_t num_slots;          // num_blocks * bs
    int64_t page_stride;
    int32_t bs;
    int32_t sanitize;
};

// Kernel launchers (return the launch's hipError_t).
hipError_t launch_decode_partial(const DecodeParams& p, int heads_per_group, int64_t grid,
                                 bool scrub, hipStream_t stream);
hipError_t launch_decode_short(const DecodeParams& p, int heads_per_group, int64_t grid,
                               bool scrub, hipStream_t stream);
size_t short_lds_bytes(int heads_per_group);
hipError_t launch_dense_partial(const DecodeParams& p, int heads_per_group, int64_t grid,
                                hipStream_t stream);
hipError_t launch_gather_dequant(const DecodeParams& p, uint16_t* kv_out, uint8_t* mask_out,
                                 bool scrub, hipStream_t stream);
// Launch shape of the split combine.  Few (token, head) rows: each row is
// cut into `slices` dim ranges, one workgroup of `waves` waves per range,
// wave w merging splits w, w + waves, ...; this spreads the partial reads
// over more compute units, each with fewer bytes in flight.  Many rows (or
// more splits than lanes in a wave): one 128-thread workgroup per row.
// The thresholds come from timing both kernels on MI355X over B*H from 64
// to 4096 and S from 4 to 64.
struct CombineShape {
    int64_t grid;
    int32_t block;
    int32_t slices;     // 0: whole-row kernel
    int32_t waves;
};
inline CombineShape combine_shape(int64_t rows, int32_t S) {
    if (S > 64 || rows >= 2048) return CombineShape{rows, kCombineThreads, 0, 0};
    const int q = rows <= 128 ? 4 : 2;
    return CombineShape{rows * q, 64 * q, q, q};
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream);

// Records `status` and a printf-style message as the calling thread's last
// error (dsv4_last_error) and returns `status`.
int set_last_error(int status, const char* fmt, ...);
hipError_t launch_convert(const ConvertParams& p, hipStream_t stream);
hipError_t launch_quantize_store(const StoreParams& p, hipStream_t stream);
hipError_t launch_gather_floor(const DecodeParams& p, int64_t grid, uint32_t* words,
                               hipStream_t stream);

}  // namespace dsv4
