// Host side of the C ABI declared in include/dsv4.h: argument validation,
// the split selector, workspace layout and kernel launches.  Nothing here
// allocates, synchronises or throws; plan and workspace queries make no HIP
// call at all, so they run on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "dsv4.h"
#include "dsv4_diag.h"
#include "internal.hpp"

namespace {

thread_local std::string g_last_error;

int vfail(int status, const char* fmt, va_list ap) {
    char buf[512];
    vsnprintf(buf, sizeof buf, fmt, ap);
    g_last_error = buf;
    return status;
}

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    const int r = vfail(status, fmt, ap);
    va_end(ap);
    return r;
}

int ok() {
    g_last_error.clear();
    return DSV4_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Shape {
    int hg;       // heads per workgroup
    int groups;   // head groups
    int splits;   // S: split slots per (token, head) row of the partials
    int bal;      // balanced splits: the split budget per token (units = B * bal); 0 = off
    bool short_kernel;
    int64_t kt;   // topk + swa
    int64_t idx_stride;
};

// Validates the descriptor and picks S.  want_ws: also check the workspace.
int make_plan(const dsv4_decode_desc* d, int32_t num_splits, Shape* sh, dsv4_plan* plan) {
    using namespace dsv4;
    if (!d) return fail(DSV4_ERR_INVALID_ARGUMENT, "desc is NULL");
    if (d->batch < 1) return fail(DSV4_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", d->batch);
    if (d->num_heads < 16 || d->num_heads > 128 || d->num_heads % 16)
        return fail(DSV4_ERR_INVALID_ARGUMENT,
                    "num_heads must be a multiple of 16 in [16, 128] (got %d)", d->num_heads);
    if (d->topk < 0 || d->swa < 0)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "topk and swa must be >= 0 (got %d, %d)", d->topk,
                    d->swa);
    const int64_t kt = (int64_t)d->topk + d->swa;
    if (kt < 1 || kt > (1 << 24))
        return fail(DSV4_ERR_INVALID_ARGUMENT, "topk + swa must lie in [1, 2^24] (got %lld)",
                    (long long)kt);
    if (d->block_size < 1)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "block_size must be >= 1 (got %d)", d->block_size);
    if (d->num_blocks < 1)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "num_blocks must be >= 1");
    if (d->page_stride < (int64_t)d->block_size * kRowBytes || d->page_stride % 8)
        return fail(DSV4_ERR_INVALID_ARGUMENT,
                    "page_stride must be a multiple of 8 and >= block_size*584 = %lld (got %lld)",
                    (long long)d->block_size * kRowBytes, (long long)d->page_stride);
    if (d->num_blocks > INT64_MAX / d->page_stride)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "num_blocks * page_stride overflows");
    if (d->tokens_per_seq < 0 || (d->tokens_per_seq > 1 && d->batch % d->tokens_per_seq))
        return fail(DSV4_ERR_INVALID_ARGUMENT,
                    "tokens_per_seq must be >= 0 and divide batch (got %d for batch %d)",
                    d->tokens_per_seq, d->batch);
    const uint32_t known = DSV4_DECODE_SCRUB | DSV4_DECODE_PIPELINED | DSV4_DECODE_BALANCE;
    if (d->flags & ~known)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "unknown decode flags 0x%x",
                    (unsigned)(d->flags & ~known));
    const int64_t idx_stride = d->topk_idx_stride == 0 ? kt : d->topk_idx_stride;
    if (idx_stride < kt)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "topk_idx_stride %lld < topk + swa %lld",
                    (long long)idx_stride, (long long)kt);

    // Heads per workgroup: a multiple of 16 that divides H, at most 64 (see
    // below for the choice between more head groups and more splits).
    if (num_splits != 0 && (num_splits < 1 || num_splits > kMaxSplits))
        return fail(DSV4_ERR_INVALID_ARGUMENT, "num_splits must be 0 (auto) or in [1, %d] (got %d)",
                    kMaxSplits, num_splits);
    // Selector split count for `groups` head groups.  want: as many splits
    // as still give every workgroup a compute unit of its own (one partial
    // workgroup fills a CU's LDS, so a grid past 256 runs a second round),
    // at most kMaxAutoSplits and at most one per tile; then the fewest
    // splits with the same tiles per split, so no split is left without
    // entries (the split chunks are whole tiles).
    const int64_t tiles = ceil_div(kt, kTile);
    auto auto_want = [&](int groups) -> int64_t {
        if (d->batch >= 256) return 1;
        int64_t want = kCUs / ((int64_t)d->batch * groups);
        if (want > kMaxAutoSplits) want = kMaxAutoSplits;
        if (want > tiles) want = tiles;
        return want < 1 ? 1 : want;
    };
    auto whole_tiles = [&](int64_t want) -> int { return (int)ceil_div(tiles, ceil_div(tiles, want)); };
    // The grouping fills the chip when one more split would not fit.
    auto fills = [&](int groups, int64_t want) {
        return (int64_t)d->batch * groups * (want + 1) > kCUs;
    };
    // With the split count left to the selector, the smallest group whose
    // splits fill the chip while each split keeps at most kMaxSplitTiles tiles
    // wins: smaller groups reach the chip with fewer splits, so less partial
    // traffic.  Otherwise (no such group, or a forced split count) the
    // largest group that fills the chip, else 16.
    int hg = 0, groups = 0, S = 0;
    if (num_splits == 0) {
        for (int cand = 16; cand <= kMaxHeadsPerGroup; cand += 16) {
            if (d->num_heads % cand) continue;
            const int g = d->num_heads / cand;
            const int64_t want = auto_want(g);
            const int sc = whole_tiles(want);
            const int64_t split_tiles = ceil_div(ceil_div(kt, sc), kTile);
            if (sc >= 2 && split_tiles <= kMaxSplitTiles && fills(g, want)) {
                hg = cand;
                groups = g;
                S = sc;
                break;
            }
        }
    }
    if (hg == 0) {
        for (int cand = kMaxHeadsPerGroup; cand >= 16; cand -= 16) {
            if (d->num_heads % cand) continue;
            hg = cand;
            groups = d->num_heads / cand;
            if (num_splits != 0) {
                S = num_splits;
                if ((int64_t)d->batch * S * groups >= kCUs) break;
            } else {
                const int64_t want = auto_want(groups);
                S = whole_tiles(want);
                if (fills(groups, want)) break;
            }
        }
    }
    const int64_t units = (int64_t)d->batch * S;
    const int64_t grid = ceil_div(units, kXcds) * kXcds * groups;
    if (grid > INT32_MAX) return fail(DSV4_ERR_INVALID_ARGUMENT, "grid too large");

    // The short-split kernel takes splits of at most kShortMaxEntries entries
    // (chunks are whole tiles, as in the kernels) with 16, 32 or 64 heads.
    const int64_t chunk_max = ceil_div(ceil_div(kt, S), kTile) * kTile;
    const bool short_kernel = chunk_max <= kShortMaxEntries && (hg == 16 || hg == 32 || hg == 64) &&
                              !(d->flags & DSV4_DECODE_PIPELINED);
    // Balanced splits: the pipelined kernel's plans with S >= 2 and at most
    // 64 tokens; the partials get S + ceil(S / 4) split slots per row so the
    // longest tokens can take more than S splits.
    const int bal = (d->flags & DSV4_DECODE_BALANCE) && !short_kernel && S >= 2 && d->batch <= 64
                        ? S
                        : 0;
    const int slots = bal ? (int)std::min<int64_t>(kMaxSplits, S + ceil_div(S, 4)) : S;
    sh->hg = hg;
    sh->groups = groups;
    sh->splits = slots;
    sh->bal = bal;
    sh->short_kernel = short_kernel;
    sh->kt = kt;
    sh->idx_stride = idx_stride;
    if (plan) {
        memset(plan, 0, sizeof *plan);
        plan->num_splits = slots;
        plan->heads_per_group = hg;
        plan->head_groups = groups;
        plan->tile_entries = kTile;
        plan->grid_partial = grid;
        plan->block_partial = kThreads;
        const dsv4::CombineShape cs =
            dsv4::combine_shape((int64_t)d->batch * d->num_heads, slots);
        plan->grid_combine = slots > 1 ? cs.grid : 0;
        plan->block_combine = slots > 1 ? cs.block : 0;
        plan->workspace_bytes =
            slots > 1
                ? (size_t)d->batch * d->num_heads * slots * (kD * sizeof(uint16_t) + sizeof(float))
                : 0;
        plan->lds_bytes = short_kernel ? short_lds_bytes(hg) : lds_bytes_for(hg);
        plan->partial_kernel = short_kernel ? DSV4_KERNEL_SHORT : DSV4_KERNEL_PIPELINED;
        plan->balanced_splits = bal;
    }
    return DSV4_OK;
}

int check_decode_ptrs(const dsv4_decode_desc* d, const dsv4_plan& plan, const void* q,
                      const void* kv, const int32_t* bt, const int32_t* idx, void* out) {
    if (!q || !kv || !idx || !out)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "q, kv_cache, topk_idx and out must not be NULL");
    if (!aligned(q, 16) || !aligned(out, 16))
        return fail(DSV4_ERR_INVALID_ARGUMENT, "q and out must be 16-byte aligned");
    if (!aligned(kv, 8)) return fail(DSV4_ERR_INVALID_ARGUMENT, "kv_cache must be 8-byte aligned");
    if (!aligned(idx, 4)) return fail(DSV4_ERR_INVALID_ARGUMENT, "topk_idx must be 4-byte aligned");
    if (bt) {
        if (d->max_blocks_per_seq < 1)
            return fail(DSV4_ERR_INVALID_ARGUMENT, "max_blocks_per_seq must be >= 1 with a block table");
        if (d->block_table_stride < d->max_blocks_per_seq)
            return fail(DSV4_ERR_INVALID_ARGUMENT, "block_table_stride %lld < max_blocks_per_seq %d",
                        (long long)d->block_table_stride, d->max_blocks_per_seq);
    }
    if (plan.workspace_bytes) {
        if (!d->workspace)
            return fail(DSV4_ERR_WORKSPACE_TOO_SMALL, "num_splits = %d needs a workspace of %zu bytes",
                        plan.num_splits, plan.workspace_bytes);
        if (d->workspace_bytes < plan.workspace_bytes)
            return fail(DSV4_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu",
                        d->workspace_bytes, plan.workspace_bytes);
        if (!aligned(d->workspace, 16))
            return fail(DSV4_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    }
    return DSV4_OK;
}

dsv4::DecodeParams make_params(const dsv4_decode_desc* d, const Shape& sh, const void* q,
                               const void* kv, const int32_t* bt, const int32_t* idx,
                               const int32_t* valid_len, const float* sink, void* out, float* lse) {
    dsv4::DecodeParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.kv = static_cast<const uint8_t*>(kv);
    p.bt = bt;
    p.idx = idx;
    p.valid_len = valid_len;
    p.mask = nullptr;
    p.kv2 = nullptr;
    p.bt2 = nullptr;
    p.num_blocks2 = p.bt_stride2 = p.page_stride2 = 0;
    p.bs2 = 1;
    p.max_blocks2 = 0;
    p.sink = sink;
    p.out = static_cast<uint16_t*>(out);
    p.lse = lse;
    const size_t n_part = (size_t)d->batch * d->num_heads * sh.splits * dsv4::kD;
    p.part_o = sh.splits > 1 ? static_cast<uint16_t*>(d->workspace) : nullptr;
    p.part_lse = sh.splits > 1
                     ? reinterpret_cast<float*>(static_cast<uint16_t*>(d->workspace) + n_part)
                     : nullptr;
    p.num_blocks = d->num_blocks;
    p.bt_stride = d->block_table_stride;
    p.page_stride = d->page_stride;
    p.idx_stride = sh.idx_stride;
    p.units = (int64_t)d->batch * (sh.bal ? sh.bal : sh.splits);
    p.B = d->batch;
    p.H = d->num_heads;
    p.topk = d->topk;
    p.swa = d->swa;
    p.bs = d->block_size;
    p.max_blocks = bt ? d->max_blocks_per_seq : 0;
    p.S = sh.splits;
    p.bal = sh.bal;
    p.bal_hi = sh.bal ? (int32_t)ceil_div(ceil_div(sh.kt, sh.bal), dsv4::kTile) : 0;
    p.G = sh.groups;
    p.sq = d->tokens_per_seq > 1 ? d->tokens_per_seq : 1;
    p.qk_scale_log2 = d->sm_scale * 1.4426950408889634f;
    p.fd_S = dsv4::make_fastdiv((uint32_t)p.S);
    p.fd_G = dsv4::make_fastdiv((uint32_t)p.G);
    p.fd_sq = dsv4::make_fastdiv((uint32_t)p.sq);
    p.fd_bs = dsv4::make_fastdiv((uint32_t)p.bs);
    p.fd_bs2 = p.fd_bs;
    p.timeline = nullptr;
    p.slots = nullptr;
    return p;
}

int launched(hipError_t e, const char* what) {
    if (e != hipSuccess)
        return fail(DSV4_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

int check_pool(const dsv4_cache_pool* pl, const char* which) {
    if (!pl || !pl->kv_cache)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "%s pool: kv_cache must not be NULL", which);
    if (!aligned(pl->kv_cache, 8))
        return fail(DSV4_ERR_INVALID_ARGUMENT, "%s pool: kv_cache must be 8-byte aligned", which);
    if (pl->block_size < 1 || pl->num_blocks < 1)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "%s pool: block_size and num_blocks must be >= 1",
                    which);
    if (pl->page_stride < (int64_t)pl->block_size * dsv4::kRowBytes || pl->page_stride % 8)
        return fail(DSV4_ERR_INVALID_ARGUMENT,
                    "%s pool: page_stride must be a multiple of 8 and >= block_size*584", which);
    if (pl->num_blocks > INT64_MAX / pl->page_stride)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "%s pool: num_blocks * page_stride overflows", which);
    if (pl->block_table &&
        (pl->max_blocks_per_seq < 1 || pl->block_table_stride < pl->max_blocks_per_seq))
        return fail(DSV4_ERR_INVALID_ARGUMENT, "%s pool: bad block-table geometry", which);
    return DSV4_OK;
}

// slots (single pool with a block table only): also write the req-local ->
// global conversion of every index column, inside the short-split kernel
// when the plan picks it, else with a conversion launch before the decode.
int decode_impl(const dsv4_decode_desc* d, const void* q, const void* kv, const int32_t* bt,
                const int32_t* idx, const int32_t* valid_len, const float* sink, void* out,
                float* lse, int32_t num_splits, hipStream_t stream, bool with_combine,
                const dsv4_cache_pool* swa_pool = nullptr, int32_t* slots = nullptr) {
    Shape sh;
    dsv4_plan plan;
    int st = make_plan(d, num_splits, &sh, &plan);
    if (st) return st;
    st = check_decode_ptrs(d, plan, q, kv, bt, idx, out);
    if (st) return st;
    dsv4::DecodeParams p = make_params(d, sh, q, kv, bt, idx, valid_len, sink, out, lse);
    if (swa_pool) {
        p.kv2 = static_cast<const uint8_t*>(swa_pool->kv_cache);
        p.bt2 = swa_pool->block_table;
        p.num_blocks2 = swa_pool->num_blocks;
        p.bt_stride2 = swa_pool->block_table_stride;
        p.page_stride2 = swa_pool->page_stride;
        p.bs2 = swa_pool->block_size;
        p.fd_bs2 = dsv4::make_fastdiv((uint32_t)p.bs2);
        p.max_blocks2 = swa_pool->block_table ? swa_pool->max_blocks_per_seq : 0;
    }
    (void)hipGetLastError();   // start from a clean error state
    if (slots) {
        // Inside the partial kernel when it can (the short-split kernel always;
        // the pipelined one with at most 1024 index columns per split), else a
        // conversion launch first.
        if (sh.short_kernel || (!sh.bal && ceil_div(sh.kt, sh.splits) <= 2 * dsv4::kThreads)) {
            p.slots = slots;
        } else {
            dsv4::ConvertParams c;
            c.req_id = nullptr;
            c.bt = bt;
            c.ti = idx;
            c.cu = nullptr;
            c.out = slots;
            c.bt_stride = d->block_table_stride;
            c.ti_stride = sh.idx_stride;
            c.num_reqs = d->batch / p.sq;
            c.max_blocks = d->max_blocks_per_seq;
            c.num_tokens = d->batch;
            c.width = (int32_t)sh.kt;
            c.bs = d->block_size;
            c.fill = -1;
            c.sq = p.sq;
            st = launched(dsv4::launch_convert(c, stream), "convert");
            if (st) return st;
        }
    }
    const bool scrub = (d->flags & DSV4_DECODE_SCRUB) != 0;
    st = sh.short_kernel && !swa_pool
             ? launched(dsv4::launch_decode_short(p, sh.hg, plan.grid_partial, scrub, stream),
                        "decode short")
             : launched(dsv4::launch_decode_partial(p, sh.hg, plan.grid_partial, scrub, stream),
                        "decode partial");
    if (st || !with_combine || sh.splits == 1) return st;
    dsv4::CombineParams c;
    c.part_o = p.part_o;
    c.part_lse = p.part_lse;
    c.sink = sink;
    c.out = p.out;
    c.lse = lse;
    c.B = d->batch;
    c.H = d->num_heads;
    c.S = sh.splits;
    return launched(dsv4::launch_combine(c, stream), "combine");
}

int decode_with_slots(const dsv4_decode_desc* desc, const void* q, const void* kv_cache,
                      const int32_t* block_table, const int32_t* topk_idx,
                      const int32_t* valid_len, const float* sink, void* out, float* lse,
                      int32_t num_splits, int32_t* global_slots, hipStream_t stream,
                      bool with_combine) {
    if (!block_table || !global_slots)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "block_table and global_slots must not be NULL");
    if (!aligned(global_slots, 4))
        return fail(DSV4_ERR_INVALID_ARGUMENT, "global_slots must be 4-byte aligned");
    return decode_impl(desc, q, kv_cache, block_table, topk_idx, valid_len, sink, out, lse,
                       num_splits, stream, with_combine, nullptr, global_slots);
}

}  // namespace

namespace dsv4 {
int set_last_error(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    const int r = vfail(status, fmt, ap);
    va_end(ap);
    return r;
}
}  // namespace dsv4

extern "C" {

const char* dsv4_status_string(int status) {
    switch (status) {
        case DSV4_OK: return "DSV4_OK";
        case DSV4_ERR_INVALID_ARGUMENT: return "DSV4_ERR_INVALID_ARGUMENT";
        case DSV4_ERR_NOT_SUPPORTED: return "DSV4_ERR_NOT_SUPPORTED";
        case DSV4_ERR_WORKSPACE_TOO_SMALL: return "DSV4_ERR_WORKSPACE_TOO_SMALL";
        case DSV4_ERR_HIP: return "DSV4_ERR_HIP";
        default: return "DSV4_ERR_UNKNOWN";
    }
}

const char* dsv4_last_error(void) { return g_last_error.c_str(); }

int dsv4_sparse_decode_plan(const dsv4_decode_desc* desc, int32_t num_splits, dsv4_plan* plan) {
    Shape sh;
    if (!plan) return fail(DSV4_ERR_INVALID_ARGUMENT, "plan is NULL");
    const int st = make_plan(desc, num_splits, &sh, plan);
    return st ? st : ok();
}

size_t dsv4_sparse_decode_workspace_bytes(const dsv4_decode_desc* desc, int32_t num_splits) {
    Shape sh;
    dsv4_plan plan;
    if (make_plan(desc, num_splits, &sh, &plan)) return 0;
    ok();
    return plan.workspace_bytes;
}

int dsv4_sparse_decode(const dsv4_decode_desc* desc, const void* q, const void* kv_cache,
                       const int32_t* block_table, const int32_t* topk_idx,
                       const int32_t* valid_len, const float* sink, void* out, float* lse,
                       int32_t num_splits, hipStream_t stream) {
    return decode_impl(desc, q, kv_cache, block_table, topk_idx, valid_len, sink, out, lse,
                       num_splits, stream, true);
}

int dsv4_sparse_decode_with_slots(const dsv4_decode_desc* desc, const void* q,
                                  const void* kv_cache, const int32_t* block_table,
                                  const int32_t* topk_idx, const int32_t* valid_len,
                                  const float* sink, void* out, float* lse, int32_t num_splits,
                                  int32_t* global_slots, hipStream_t stream) {
    return decode_with_slots(desc, q, kv_cache, block_table, topk_idx, valid_len, sink, out, lse,
                             num_splits, global_slots, stream, true);
}

int dsv4_sparse_decode_partial_with_slots(const dsv4_decode_desc* desc, const void* q,
                                          const void* kv_cache, const int32_t* block_table,
                                          const int32_t* topk_idx, const int32_t* valid_len,
                                          const float* sink, void* out, float* lse,
                                          int32_t num_splits, int32_t* global_slots,
                                          hipStream_t stream) {
    return decode_with_slots(desc, q, kv_cache, block_table, topk_idx, valid_len, sink, out, lse,
                             num_splits, global_slots, stream, false);
}

int dsv4_gather_floor(const dsv4_decode_desc* desc, const void* kv_cache,
                      const int32_t* block_table, const int32_t* topk_idx,
                      const int32_t* valid_len, int32_t num_splits, uint32_t* words,
                      hipStream_t stream) {
    Shape sh;
    dsv4_plan plan;
    int st = make_plan(desc, num_splits, &sh, &plan);
    if (st) return st;
    if (sh.bal)
        return fail(DSV4_ERR_INVALID_ARGUMENT,
                    "the gather floor takes the uniform split plan (no DSV4_DECODE_BALANCE)");
    if (!kv_cache || !topk_idx || !words)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "kv_cache, topk_idx and words must not be NULL");
    if (block_table) {
        if (desc->max_blocks_per_seq < 1)
            return fail(DSV4_ERR_INVALID_ARGUMENT, "max_blocks_per_seq must be >= 1 with a block table");
        if (desc->block_table_stride < desc->max_blocks_per_seq)
            return fail(DSV4_ERR_INVALID_ARGUMENT, "block_table_stride < max_blocks_per_seq");
    }
    const dsv4::DecodeParams p = make_params(desc, sh, nullptr, kv_cache, block_table, topk_idx,
                                             valid_len, nullptr, nullptr, nullptr);
    (void)hipGetLastError();
    return launched(dsv4::launch_gather_floor(p, plan.grid_partial, words, stream), "gather floor");
}

int dsv4_short_timeline(const dsv4_decode_desc* desc, const void* q, const void* kv_cache,
                        const int32_t* block_table, const int32_t* topk_idx,
                        const int32_t* valid_len, const float* sink, void* out, float* lse,
                        int32_t num_splits, uint64_t* stamps, hipStream_t stream) {
    Shape sh;
    dsv4_plan plan;
    int st = make_plan(desc, num_splits, &sh, &plan);
    if (st) return st;
    if (!sh.short_kernel || (desc->flags & DSV4_DECODE_SCRUB))
        return fail(DSV4_ERR_NOT_SUPPORTED,
                    "the timeline covers the short-split kernel without scrub only");
    if (!stamps) return fail(DSV4_ERR_INVALID_ARGUMENT, "stamps must not be NULL");
    st = check_decode_ptrs(desc, plan, q, kv_cache, block_table, topk_idx, out);
    if (st) return st;
    dsv4::DecodeParams p = make_params(desc, sh, q, kv_cache, block_table, topk_idx, valid_len,
                                       sink, out, lse);
    p.timeline = stamps;
    (void)hipGetLastError();
    return launched(dsv4::launch_decode_short(p, sh.hg, plan.grid_partial, false, stream),
                    "decode short (timeline)");
}

int dsv4_sparse_decode_partial(const dsv4_decode_desc* desc, const void* q,
                               const void* kv_cache, const int32_t* block_table,
                               const int32_t* topk_idx, const int32_t* valid_len,
                               const float* sink, void* out, float* lse, int32_t num_splits,
                               hipStream_t stream) {
    return decode_impl(desc, q, kv_cache, block_table, topk_idx, valid_len, sink, out, lse,
                       num_splits, stream, false);
}

int dsv4_combine_splits(int32_t batch, int32_t num_heads, int32_t num_splits,
                        const void* part_out, const float* part_lse, const float* sink,
                        void* out, float* lse, hipStream_t stream) {
    if (batch < 1 || num_heads < 1 || num_splits < 1)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "batch, num_heads and num_splits must be >= 1");
    if ((int64_t)batch * num_heads > INT32_MAX)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "batch * num_heads too large");
    if (!part_out || !part_lse || !out)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "part_out, part_lse and out must not be NULL");
    if (!aligned(part_out, 8) || !aligned(out, 8) || !aligned(part_lse, 4))
        return fail(DSV4_ERR_INVALID_ARGUMENT,
                    "part_out and out must be 8-byte aligned, part_lse 4-byte aligned");
    dsv4::CombineParams c;
    c.part_o = static_cast<const uint16_t*>(part_out);
    c.part_lse = part_lse;
    c.sink = sink;
    c.out = static_cast<uint16_t*>(out);
    c.lse = lse;
    c.B = batch;
    c.H = num_heads;
    c.S = num_splits;
    (void)hipGetLastError();
    return launched(dsv4::launch_combine(c, stream), "combine");
}

int dsv4_convert_req_index_to_global(const int32_t* req_id, int32_t num_reqs,
                                     const int32_t* block_table, int64_t bt_stride,
                                     int32_t max_blocks_per_req, const int32_t* token_indices,
                                     int64_t ti_stride, int32_t num_tokens, int32_t width,
                                     int32_t block_size, const int32_t* cu_seqlens,
                                     int32_t invalid_fill, int32_t* out, hipStream_t stream) {
    if (num_tokens < 0 || width < 0)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "num_tokens and width must be >= 0");
    if (num_tokens == 0 || width == 0) return ok();
    if (!block_table || !token_indices || !out)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "block_table, token_indices and out must not be NULL");
    if (block_size < 1) return fail(DSV4_ERR_INVALID_ARGUMENT, "block_size must be >= 1");
    if (num_reqs < 0 || max_blocks_per_req < 0)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "num_reqs and max_blocks_per_req must be >= 0");
    if (bt_stride < max_blocks_per_req)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "bt_stride < max_blocks_per_req");
    if (ti_stride < width) return fail(DSV4_ERR_INVALID_ARGUMENT, "ti_stride < width");
    dsv4::ConvertParams p;
    p.req_id = req_id;
    p.bt = block_table;
    p.ti = token_indices;
    p.cu = cu_seqlens;
    p.out = out;
    p.bt_stride = bt_stride;
    p.ti_stride = ti_stride;
    p.num_reqs = num_reqs;
    p.max_blocks = max_blocks_per_req;
    p.num_tokens = num_tokens;
    p.width = width;
    p.bs = block_size;
    p.fill = invalid_fill;
    p.sq = 1;
    (void)hipGetLastError();
    return launched(dsv4::launch_convert(p, stream), "convert");
}

uint32_t dsv4_decode_flags_for_cache(int32_t cache_is_fp8_ds_mla, int32_t has_kv_transfer,
                                     int32_t has_extra_cache, int32_t writer_sanitizes) {
    const bool trusted = cache_is_fp8_ds_mla && !has_kv_transfer && has_extra_cache &&
                         writer_sanitizes;
    return trusted ? 0u : DSV4_DECODE_SCRUB;
}

int dsv4_gather_dequant(const dsv4_decode_desc* desc, const void* kv_cache,
                        const int32_t* block_table, const int32_t* topk_idx,
                        const int32_t* valid_len, void* kv_out, uint8_t* mask_out,
                        hipStream_t stream) {
    Shape sh;
    dsv4_plan plan;
    int st = make_plan(desc, 1, &sh, &plan);
    if (st) return st;
    if (!kv_cache || !topk_idx || !kv_out || !mask_out)
        return fail(DSV4_ERR_INVALID_ARGUMENT,
                    "kv_cache, topk_idx, kv_out and mask_out must not be NULL");
    if (!aligned(kv_cache, 8)) return fail(DSV4_ERR_INVALID_ARGUMENT, "kv_cache must be 8-byte aligned");
    if (!aligned(kv_out, 16)) return fail(DSV4_ERR_INVALID_ARGUMENT, "kv_out must be 16-byte aligned");
    if (block_table && (desc->max_blocks_per_seq < 1 ||
                        desc->block_table_stride < desc->max_blocks_per_seq))
        return fail(DSV4_ERR_INVALID_ARGUMENT, "bad block-table geometry");
    if ((int64_t)desc->batch * ((sh.kt + dsv4::kTile - 1) / dsv4::kTile) > INT32_MAX)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "batch * entries too large");
    dsv4::DecodeParams p = make_params(desc, sh, nullptr, kv_cache, block_table, topk_idx,
                                       valid_len, nullptr, nullptr, nullptr);
    (void)hipGetLastError();
    return launched(dsv4::launch_gather_dequant(p, static_cast<uint16_t*>(kv_out), mask_out,
                                                (desc->flags & DSV4_DECODE_SCRUB) != 0, stream),
                    "gather dequant");
}

int dsv4_dense_decode(const dsv4_decode_desc* desc, const void* q, const void* kv_dense,
                      const uint8_t* mask, const float* sink, void* out, float* lse,
                      int32_t num_splits, hipStream_t stream) {
    Shape sh;
    dsv4_plan plan;
    int st = make_plan(desc, num_splits, &sh, &plan);
    if (st) return st;
    if (desc->flags)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "dense decode takes no flags (scrub applies when "
                                               "gathering)");
    if (!q || !kv_dense || !mask || !out)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "q, kv_dense, mask and out must not be NULL");
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(kv_dense, 16))
        return fail(DSV4_ERR_INVALID_ARGUMENT, "q, kv_dense and out must be 16-byte aligned");
    if (plan.workspace_bytes) {
        if (!desc->workspace || desc->workspace_bytes < plan.workspace_bytes)
            return fail(DSV4_ERR_WORKSPACE_TOO_SMALL, "num_splits = %d needs a workspace of %zu bytes",
                        plan.num_splits, plan.workspace_bytes);
        if (!aligned(desc->workspace, 16))
            return fail(DSV4_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    }
    // Dense rows: every token has kt entries, all in one effective list.
    dsv4::DecodeParams p = make_params(desc, sh, q, kv_dense, nullptr, nullptr, nullptr, sink, out,
                                       lse);
    p.mask = mask;
    p.topk = (int32_t)sh.kt;
    p.swa = 0;
    p.idx_stride = sh.kt;
    p.sq = 1;
    p.max_blocks = 0;
    (void)hipGetLastError();
    st = launched(dsv4::launch_dense_partial(p, sh.hg, plan.grid_partial, stream), "dense partial");
    if (st || sh.splits == 1) return st;
    dsv4::CombineParams c;
    c.part_o = p.part_o;
    c.part_lse = p.part_lse;
    c.sink = sink;
    c.out = p.out;
    c.lse = lse;
    c.B = desc->batch;
    c.H = desc->num_heads;
    c.S = sh.splits;
    return launched(dsv4::launch_combine(c, stream), "combine");
}

int dsv4_sparse_decode_dual(const dsv4_decode_desc* desc, const void* q,
                            const dsv4_cache_pool* main_pool, const dsv4_cache_pool* swa_pool,
                            const int32_t* topk_idx, const int32_t* valid_len, const float* sink,
                            void* out, float* lse, int32_t num_splits, hipStream_t stream) {
    if (!desc) return fail(DSV4_ERR_INVALID_ARGUMENT, "desc must not be NULL");
    int st = check_pool(main_pool, "main");
    if (st) return st;
    st = check_pool(swa_pool, "swa");
    if (st) return st;
    if ((main_pool->block_table == nullptr) != (swa_pool->block_table == nullptr))
        return fail(DSV4_ERR_INVALID_ARGUMENT,
                    "both pools need a block table, or neither (global slots)");
    dsv4_decode_desc d = *desc;
    d.block_size = main_pool->block_size;
    d.num_blocks = main_pool->num_blocks;
    d.page_stride = main_pool->page_stride;
    d.block_table_stride = main_pool->block_table_stride;
    d.max_blocks_per_seq = main_pool->max_blocks_per_seq;
    return decode_impl(&d, q, main_pool->kv_cache, main_pool->block_table, topk_idx, valid_len,
                       sink, out, lse, num_splits, stream, true, swa_pool);
}

int dsv4_quantize_store(const void* rows, int64_t row_stride, const int64_t* slot_mapping,
                        int64_t num_rows, void* kv_cache, int32_t block_size, int64_t num_blocks,
                        int64_t page_stride, uint32_t flags, hipStream_t stream) {
    if (num_rows < 0) return fail(DSV4_ERR_INVALID_ARGUMENT, "num_rows must be >= 0");
    if (flags & ~DSV4_STORE_SANITIZE)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "unknown store flags 0x%x",
                    (unsigned)(flags & ~DSV4_STORE_SANITIZE));
    if (block_size < 1) return fail(DSV4_ERR_INVALID_ARGUMENT, "block_size must be >= 1");
    if (num_blocks < 1) return fail(DSV4_ERR_INVALID_ARGUMENT, "num_blocks must be >= 1");
    if (page_stride < (int64_t)block_size * dsv4::kRowBytes || page_stride % 8)
        return fail(DSV4_ERR_INVALID_ARGUMENT,
                    "page_stride must be a multiple of 8 and >= block_size*584 = %lld (got %lld)",
                    (long long)block_size * dsv4::kRowBytes, (long long)page_stride);
    if (num_blocks > INT64_MAX / page_stride)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "num_blocks * page_stride overflows");
    if (row_stride < dsv4::kD || row_stride % 8)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "row_stride must be a multiple of 8 and >= 512");
    if (num_rows == 0) return ok();
    if (!rows || !slot_mapping || !kv_cache)
        return fail(DSV4_ERR_INVALID_ARGUMENT, "rows, slot_mapping and kv_cache must not be NULL");
    if (!aligned(rows, 16)) return fail(DSV4_ERR_INVALID_ARGUMENT, "rows must be 16-byte aligned");
    if (!aligned(slot_mapping, 8))
        return fail(DSV4_ERR_INVALID_ARGUMENT, "slot_mapping must be 8-byte aligned");
    if (!aligned(kv_cache, 8)) return fail(DSV4_ERR_INVALID_ARGUMENT, "kv_cache must be 8-byte aligned");
    if ((num_rows + 3) / 4 > INT32_MAX) return fail(DSV4_ERR_INVALID_ARGUMENT, "num_rows too large");
    dsv4::StoreParams p;
    p.rows = static_cast<const uint16_t*>(rows);
    p.slots = slot_mapping;
    p.kv = static_cast<uint8_t*>(kv_cache);
    p.n = num_rows;
    p.row_stride = row_stride;
    p.num_blocks = num_blocks;
    p.num_slots = num_blocks * block_size;
    p.page_stride = page_stride;
    p.bs = block_size;
    p.sanitize = (flags & DSV4_STORE_SANITIZE) ? 1 : 0;
    (void)hipGetLastError();
    return launched(dsv4::launch_quantize_store(p, stream), "quantize store");
}

}  // extern "C"
