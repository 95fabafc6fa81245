// Sparse FP8 MLA decode kernels for gfx950 (CDNA4): the partial (split-K)
// kernel, the log-sum-exp combine kernel, the two-kernel path's gather and
// dense-source kernels, and the gather-floor measurement kernel.
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
// walks its slice of the token's entry list in tiles of 32 cache rows, as a
// software pipeline with one barrier per step.  In step t:
//   * waves 0..HG/16-1 ("consumers", one per 16-head MFMA tile) run QK of tile t
//     on bf16 MFMA 16x16x32 (q held in registers, S^T = K q^T so each lane
//     holds 8 scores of one head) fused with the online softmax (cross-row
//     permlane reductions, lazy rescaling: the running max only moves when a
//     score exceeds it by more than 2^8), writing bf16 probabilities;
//   * waves 4..7 ("producers", 8 lanes per cache row) dequantise tile t+1
//     (FP8 x 2^(code-127) -> bf16 in one scaled convert per 2 values) into
//     one of three LDS K buffers and issue the loads of tile t+4, keeping three
//     tiles of raw bytes in flight in registers;
//   * all 8 waves run PV of tile t-1 on bf16 MFMA, wave w owning output dims
//     [64w, 64w+64); the V operand comes straight from the K tile through
//     the gfx950 LDS transpose read, so no transposed copy is kept.
// Entry resolution (index -> page via the block table -> row addresses) of
// the first 32 tiles happens up front, into an LDS ring with a per-tile
// bit mask of the rows that take part; longer splits resolve 16 more tiles
// at a time inside the loop.  Rows that take no part read a zero row, so a
// NaN in the cache can never reach an MFMA.  The running sum takes the fp32
// probabilities, the PV operand their bf16 rounding.  With one split the
// epilogue folds the sink in and writes bf16 output and lse; with several it
// writes the split's normalised bf16 partial and lse.  Output rows are staged
// in LDS and leave as whole 1 KB rows (16-byte nontemporal stores).
// Work units are (token, split) pairs; with balanced splits each token's
// split count follows its run-time length (balanced_unit below).
// Variants of the same body: SCRUB zeroes non-finite dequantised elements;
// DENSE reads already gathered bf16 rows with a mask (two tiles in flight, as
// a 1 KB row needs 32 registers per producer lane); a dual cache resolves
// the SWA entries through a second pool, chosen per entry.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "decode_common.hpp"
#include "device_util.hpp"
#include "internal.hpp"

namespace dsv4 {

// Balanced splits (the batch's tokens in the lanes of one wave, B <= 64):
// token t has eff_t = valid_len + swa entries and gets n_t = max(1,
// ceil(eff_t / (32 T))) splits of at most T tiles, with T the fewest tiles
// for which sum_t n_t stays within the budget B * bal and no n_t exceeds the
// S split slots (T = ceil(ceil((topk + swa) / bal) / 32) always qualifies).
// Work unit u is split u - (n_0 + ... + n_{t-1}) of the token t whose range
// holds it; units past the last token's splits have no work.  Every wave
// computes the same assignment.  (vLLM PR #52212 page, implementation item
// 2: a fixed grid whose rows pick their active splits at run time.)
// ceil(a / d) for 0 <= a <= 2^24 and 32 <= d < 2^24: a and d are exact in
// fp32 and a/d <= 2^19, so the quotient from the fp32 reciprocal (relative
// error below 2^-21) is within one of the exact one, and one integer
// correction step fixes it.
__device__ __forceinline__ int ceil_div_small(int a, int d) {
    int q = (int)((float)a * __builtin_amdgcn_rcpf((float)d));
    int r = a - q * d;
    if (r < 0) {
        --q;
        r += d;
    } else if (r >= d) {
        ++q;
        r -= d;
    }
    return q + (r > 0);
}

__device__ __forceinline__ bool balanced_unit(const DecodeParams& p, int unit, int lane, int& b,
                                              int& s, int& nsplit, int& vl_b) {
    // Wave reductions on DPP rows and permlane swaps, carried in fp32: every
    // value here is an integer of at most 2^24 (the plan bounds topk + swa),
    // so the sums and maxima are exact.
    auto wsum = [](int v) { return (int)xrow_sum4(row_sum16((float)v)); };
    int eff = 0;
    if (lane < p.B) {
        const int vl = p.valid_len
                           ? min(max(p.valid_len[fdiv((uint32_t)lane, p.fd_sq)], 0), p.topk)
                           : p.topk;
        eff = vl + p.swa;
    }
    const int emax = (int)xrow_max4(row_max16((float)eff));
    int lo = max(1, ceil_div_small(emax, kTile * p.S));
    int hi = p.bal_hi;
    const int budget = p.B * p.bal;
    auto splits_at = [&](int t) { return lane < p.B ? max(1, ceil_div_small(eff, kTile * t)) : 0; };
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (wsum(splits_at(mid)) <= budget)
            hi = mid;
        else
            lo = mid + 1;
    }
    const int n = splits_at(lo);
    // Inclusive prefix sum over the lanes: within each 16-lane row by DPP
    // row shifts (lanes shifted in from outside the row read 0), then the
    // totals of the rows below added from lanes 15, 31 and 47.
    float x = (float)n;
    x += dpp<0x111>(x);
    x += dpp<0x112>(x);
    x += dpp<0x114>(x);
    x += dpp<0x118>(x);
    const int xi = __builtin_bit_cast(int, x);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 15));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 31));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 47));
    const int row = lane >> 4;
    const int incl = (int)(x + (row >= 1 ? r0 : 0.f) + (row >= 2 ? r1 : 0.f) + (row >= 3 ? r2 : 0.f));
    const uint64_t past = __builtin_amdgcn_ballot_w64(lane < p.B && incl > unit);
    if (past == 0) return false;
    const int t = (int)__builtin_ctzll(past);
    nsplit = __builtin_amdgcn_readlane(n, t);
    s = unit - (__builtin_amdgcn_readlane(incl, t) - nsplit);
    b = t;
    vl_b = __builtin_amdgcn_readlane(eff, t) - p.swa;   // no second load of the length
    // Holds by construction; kept so that no index can leave the row's slots.
    return s >= 0 && s < nsplit && nsplit <= p.S;
}

// The partial kernel's body.  SCRUB: non-finite dequantised elements read
// as 0.  DENSE: rows come from a gathered bf16 buffer [B, idx_stride, 512]
// with a per-entry mask (1 = takes no part) instead of the FP8 cache.
// EMIT (block table, single pool): the workgroups of head group 0 also write
// the req-local -> global conversion of the token's index row into p.slots
// (vLLM PR #41217 report, key source snippets: the conversion kernel), split
// s taking columns [s*cc, s*cc + cc), cc = ceil((topk + swa) / S) <= 1024,
// two per thread, with loads issued beside the resolution's own.
template <int HG, bool SCRUB, bool DENSE, bool EMIT = false>
__device__ __forceinline__ void decode_partial_body(const DecodeParams& p) {
    static_assert(!(EMIT && DENSE), "the conversion output needs the FP8 cache's table");
    constexpr int MT = HG / 16;              // 16-head MFMA tiles; consumer wave w owns tile w
    static_assert(HG % 16 == 0 && HG <= kMaxHeadsPerGroup, "head group");
    using L = Smem<HG>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[L::bytes];
    __bf16* Kn = reinterpret_cast<__bf16*>(smem + L::kn);          // [3][32][512], swizzled
    __bf16* Pb = reinterpret_cast<__bf16*>(smem + L::pb);          // [2][HG][40]
    float* alpha_s = reinterpret_cast<float*>(smem + L::alpha);    // [2][HG]
    float* fin = reinterpret_cast<float*>(smem + L::fin);
    int* flags = reinterpret_cast<int*>(smem + L::flags);          // [2][4]
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
    int b, s, nsplit;                         // token, split, the token's split count
    int vl = -1;                              // the token's valid length, once known
    if (!DENSE && p.bal) {
        if (!balanced_unit(p, (int)unit, lane, b, s, nsplit, vl)) return;
    } else {
        b = (int)(unit / p.S);
        s = (int)(unit % p.S);
        nsplit = p.S;
    }
    const int seq = b / p.sq;                 // tokens of one sequence share its table and length
    const int h0 = g * HG;

    // This split's slice of the effective list main[0:vl] ++ swa, in chunks
    // rounded up to whole tiles.
    if (vl < 0) vl = p.valid_len ? min(max(p.valid_len[seq], 0), p.topk) : p.topk;
    const int eff = vl + p.swa;
    int chunk = (eff + nsplit - 1) / nsplit;
    chunk = (chunk + kTile - 1) / kTile * kTile;
    const int lo = min(s * chunk, eff);
    const int hi = min(lo + chunk, eff);
    const int ntiles = (hi - lo + kTile - 1) / kTile;

    const bool consumer = wave < MT;
    const bool producer = wave >= 4;
    // Producer: tile row and chunk lane.
    const int prow = 8 * (wave - 4) + (lane >> 4) + 4 * ((lane >> 3) & 1), l8 = lane & 7;
    const int hc = 16 * wave + l16;              // consumer lane's head (within the group)
    auto meta_tile = [&](int t) { return meta + (t % kMetaTiles) * kTile * 2; };
    auto kbuf = [&](int t) { return Kn + (t % kKBufs) * (kTile * kD); };
    // LDS fragment offsets (elements) split into a per-lane part, fixed for
    // the kernel, and the K buffer's offset, held in a scalar register, so
    // that each fragment address costs one add per step.  QK: k-steps ks and
    // ks + 8 differ by 256 elements, rows 16 + r and r by 16 rows (the
    // swizzle only moves unit bits 1-4 and depends on row bits 0-3).
    int kq[8], kvo[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) kq[i] = kofs(l16, 32 * i + 8 * lg);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
        kvo[nt] = kofs(4 * lg + (l16 >> 2), 64 * wave + 16 * nt + 4 * (l16 & 3));
    auto kbase = [&](int t) __attribute__((always_inline)) {
        int kb = (t % kKBufs) * (kTile * kD);
        asm volatile("" : "+s"(kb));
        return kb;
    };

    // One 64-register array per lane, used by role: consumers keep the q
    // row of their head in it (lane (l16, lg) holds dims 32*ks + 8*lg .. +7
    // of head 16*wave + l16 in rr[4ks..4ks+3], the B operand of QK);
    // producers keep three tiles of raw bytes in it (rr[0..59]).
    uint32_t rr[64];
    float sink_l2 = -INFINITY;                   // consumer lane's sink, base-2 units

    // q row of the consumer lane's head into rr (see above).
    auto load_q = [&]() __attribute__((always_inline)) {
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
    };

    // Resolution of the first 32 tiles (the whole ring): two entries per
    // thread, then a per-tile bit mask of the rows that take part (wave w
    // covers tiles 2w, 2w+1 and 16+2w, 17+2w).  Later tiles are resolved 16 at
    // a time inside the loop, which only splits longer than 32 tiles reach.
    // Consumer waves issue their q loads right after the block-table loads,
    // so q streams in during the table round trip (issued before the index
    // loads it would hold them back: loads retire in order).
    {
        uint64_t b0, b1;
        if constexpr (DENSE) {
            const bool v0 = dense_live(p, b, lo, hi, lo + tid);
            const bool v1 = dense_live(p, b, lo, hi, lo + kThreads + tid);
            write_dense_meta(p, meta + 2 * tid, b, lo + tid, v0);
            write_dense_meta(p, meta + 2 * (kThreads + tid), b, lo + kThreads + tid, v1);
            b0 = __builtin_amdgcn_ballot_w64(v0);
            b1 = __builtin_amdgcn_ballot_w64(v1);
        } else {
            // Conversion columns of this thread (EMIT), loaded unconditionally
            // and before the ring entries, so both sets arrive in one round trip.
            const int kt = p.topk + p.swa;
            int col0 = 0, col1 = 0;
            bool on0 = false, on1 = false;
            int32_t ci0 = -1, ci1 = -1;
            if constexpr (EMIT) {
                const int cc = (kt + p.S - 1) / p.S;
                col0 = s * cc + tid;
                col1 = col0 + kThreads;
                on0 = g == 0 && tid < cc && col0 < kt;
                on1 = g == 0 && tid + kThreads < cc && col1 < kt;
                const int32_t* row = p.idx + (int64_t)b * p.idx_stride;
                const int32_t v0 = row[on0 ? col0 : 0];
                const int32_t v1 = row[on1 ? col1 : 0];
                ci0 = on0 ? v0 : -1;
                ci1 = on1 ? v1 : -1;
            }
            const int32_t i0 = load_index(p, b, vl, hi, lo + tid);
            const int32_t i1 = load_index(p, b, vl, hi, lo + kThreads + tid);
            const Pool pl0 = pool_of(p, lo + tid >= vl);
            const Pool pl1 = pool_of(p, lo + kThreads + tid >= vl);
            // All table loads of the block (ring entries and conversion
            // columns) are issued before any is used: one round trip.  The
            // slot-writing variant always has a table.
            int32_t w0 = 0, w1 = 0, cw0 = 0, cw1 = 0;
            if (EMIT || p.bt) {
                w0 = pl0.bt[(int64_t)seq * pl0.bt_stride + table_column(pl0, i0)];
                w1 = pl1.bt[(int64_t)seq * pl1.bt_stride + table_column(pl1, i1)];
                if constexpr (EMIT) {
                    const Pool pm = pool_of(p, false);
                    cw0 = p.bt[(int64_t)seq * p.bt_stride + table_column(pm, ci0)];
                    cw1 = p.bt[(int64_t)seq * p.bt_stride + table_column(pm, ci1)];
                }
            }
            if (consumer) load_q();
            const int64_t g0 = page_from_word(p, pl0, i0, w0);
            const int64_t g1 = page_from_word(p, pl1, i1, w1);
            if constexpr (EMIT) {
                // The conversion's rule: a negative index, a block past the
                // table, a negative page entry or a slot past INT32_MAX give -1.
                auto emit = [&](int32_t ci, int32_t w, int col, bool on)
                                __attribute__((always_inline)) {
                    const bool ok = ci >= 0;
                    const int64_t blk = (ok ? ci : 0) / p.bs;
                    const bool inb = ok && blk < p.max_blocks;
                    const int64_t gs = (int64_t)w * p.bs + (ok ? ci : 0) % p.bs;
                    if (on)
                        p.slots[(int64_t)b * kt + col] =
                            inb && w >= 0 && gs <= (int64_t)INT32_MAX ? (int32_t)gs : -1;
                };
                emit(ci0, cw0, col0, on0);
                emit(ci1, cw1, col1, on1);
            }
            write_meta(pl0, meta + 2 * tid, g0, i0);
            write_meta(pl1, meta + 2 * (kThreads + tid), g1, i1);
            b0 = __builtin_amdgcn_ballot_w64(g0 >= 0);
            b1 = __builtin_amdgcn_ballot_w64(g1 >= 0);
        }
        if (lane == 0) {
            vmask[2 * wave] = (uint32_t)b0;
            vmask[2 * wave + 1] = (uint32_t)(b0 >> 32);
            vmask[kHalfTiles + 2 * wave] = (uint32_t)b1;
            vmask[kHalfTiles + 2 * wave + 1] = (uint32_t)(b1 >> 32);
        }
    }
    __syncthreads();

    // Dense rows: q is loaded beside the producers' first row loads.  The
    // sink (used at the finish) is loaded here, after the resolution: a load
    // under a branch makes the compiler wait for every older load at the join.
    if constexpr (DENSE) {
        if (consumer) load_q();
    }
    if (consumer && p.sink) sink_l2 = p.sink[h0 + hc] * kLog2e;

    if (producer) {
        if constexpr (DENSE) {
            load_dense<0>(dense_src(meta_tile(0), prow, ntiles > 0), l8, rr);
            load_dense<32>(dense_src(meta_tile(1), prow, ntiles > 1), l8, rr);
            gbyte* a2 = dense_src(meta_tile(2), prow, ntiles > 2);
            store_dense<0>(rr, prow, l8, kbuf(0));
            load_dense<0>(a2, l8, rr);
        } else {
            load_patch<0>(patch_src(meta_tile(0), prow, ntiles > 0), l8, rr);
            load_patch<20>(patch_src(meta_tile(1), prow, ntiles > 1), l8, rr);
            load_patch<40>(patch_src(meta_tile(2), prow, ntiles > 2), l8, rr);
            const PatchSrc a3 = patch_src(meta_tile(3), prow, ntiles > 3);
            store_patch<0, SCRUB>(rr, prow, l8, kbuf(0));
            load_patch<0>(a3, l8, rr);
        }
    }
    __syncthreads();

    // Online-softmax state of a consumer lane's head, in base-2 units: the
    // running max is replicated over the lane's four 16-lane rows; the running
    // sum is the lane's own share (all rows of a head rescale by the same
    // factor), summed over the rows once, before the finish.
    float m_run = -INFINITY, l_run = 0.f;
    // PV accumulators: wave w owns output dims [64w, 64w+64).  acc[mt][nt]
    // is a 16-dim x 16-head block of O^T; lane (l16, lg) holds head 16mt + l16
    // at dims 64w + 16nt + 4lg + r, r = 0..3.
    f32x4 acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Staged resolution of the next half (16 tiles, from tile 32 on) by
    // waves 0..3, two entries per lane: entry 128w + l (tiles 4w, 4w+1) and 128w + 64 + l
    // (tiles 4w+2, 4w+3).  Phase 0 loads the raw indices, phase 1 masks them
    // and loads the raw block-table entries, phase 2 turns them into pages and
    // publishes the offsets and tile masks; each load's result is first used
    // one step (one barrier) after it is issued.
    int32_t r_i0 = 0, r_i1 = 0, r_p0 = 0, r_p1 = 0;
    auto raw_index = [&](int pos) {
        const int cpos = pos < hi ? pos : lo;
        const int col = cpos < vl ? cpos : p.topk + (cpos - vl);
        return p.idx[(int64_t)b * p.idx_stride + (pos < hi ? col : 0)];
    };
    auto resolve_stage = [&](int t) __attribute__((always_inline)) {
        const int ph = t % kHalfTiles;
        const int nxt = t - ph + kHalfTiles;      // first tile of the next half
        if (nxt < kMetaTiles || nxt >= ntiles || ph >= 3) return;
        const int e0 = lo + nxt * kTile + 128 * wave + lane;
        if constexpr (DENSE) {
            // Phase 0 loads the two mask bytes, phase 2 publishes.
            if (ph == 0) {
                r_i0 = dense_live(p, b, lo, hi, e0);
                r_i1 = dense_live(p, b, lo, hi, e0 + 64);
            } else if (ph == 2) {
                int64_t* m = meta_tile(nxt) + 2 * (128 * wave + lane);
                write_dense_meta(p, m, b, e0, r_i0 != 0);
                write_dense_meta(p, m + 2 * 64, b, e0 + 64, r_i1 != 0);
                const uint64_t b0 = __builtin_amdgcn_ballot_w64(r_i0 != 0);
                const uint64_t b1 = __builtin_amdgcn_ballot_w64(r_i1 != 0);
                if (lane == 0) {
                    uint32_t* vmk = vmask + (nxt + 4 * wave) % kMetaTiles;
                    vmk[0] = (uint32_t)b0;
                    vmk[1] = (uint32_t)(b0 >> 32);
                    vmk[2] = (uint32_t)b1;
                    vmk[3] = (uint32_t)(b1 >> 32);
                }
            }
            return;
        }
        if (ph == 0) {
            r_i0 = raw_index(e0);
            r_i1 = raw_index(e0 + 64);
        } else if (ph == 1) {
            r_i0 = e0 < hi ? r_i0 : -1;
            r_i1 = e0 + 64 < hi ? r_i1 : -1;
            if (p.bt) {
                const Pool pl0 = pool_of(p, e0 >= vl), pl1 = pool_of(p, e0 + 64 >= vl);
                r_p0 = pl0.bt[(int64_t)seq * pl0.bt_stride + table_column(pl0, r_i0)];
                r_p1 = pl1.bt[(int64_t)seq * pl1.bt_stride + table_column(pl1, r_i1)];
            }
        } else {
            const Pool pl0 = pool_of(p, e0 >= vl), pl1 = pool_of(p, e0 + 64 >= vl);
            const int64_t pg0 = page_from_word(p, pl0, r_i0, r_p0), pg1 = page_from_word(p, pl1, r_i1, r_p1);
            int64_t* m = meta_tile(nxt) + 2 * (128 * wave + lane);
            write_meta(pl0, m, pg0, r_i0);
            write_meta(pl1, m + 2 * 64, pg1, r_i1);
            const uint64_t b0 = __builtin_amdgcn_ballot_w64(pg0 >= 0);
            const uint64_t b1 = __builtin_amdgcn_ballot_w64(pg1 >= 0);
            if (lane == 0) {
                uint32_t* vmk = vmask + (nxt + 4 * wave) % kMetaTiles;
                vmk[0] = (uint32_t)b0;
                vmk[1] = (uint32_t)(b0 >> 32);
                vmk[2] = (uint32_t)b1;
                vmk[3] = (uint32_t)(b1 >> 32);
            }
        }
    };

    // PV of tile k (all waves): O^T += V^T P^T with V = the K tile.  The k
    // index of the MFMA runs over the tile's entries in the order a QK lane
    // holds them: k = 8g + i is entry 4g + i (i < 4) or 16 + 4g + i - 4.  The
    // B operand (P^T) is then the QK lane's 8 probabilities as written; the A
    // operand (V^T, rows = 16 dims) comes from the K tile through the LDS
    // transpose read: lane j of 16-lane group g addresses entry 4g + j/4 (and
    // 16 + 4g + j/4) at dims base + 4(j%4), so lane i receives dim base + i
    // of entries 4g .. 4g+3 (16 + 4g .. 16 + 4g+3).
    // Rescale of the accumulators before PV of tile k (rare: only when a
    // consumer moved its running max in tile k), kept apart from the MFMA
    // part so the latter sits in one basic block with the consumers' softmax.
    auto pv_rescale = [&](int k) __attribute__((always_inline)) {
        const int* fl = flags + (k & 1) * 4;
        bool rescale = false;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) rescale |= fl[mt] != 0;
        if (rescale) {
            const float* al = alpha_s + (k & 1) * HG;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float a = al[16 * mt + l16];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) acc[mt][nt] *= a;
            }
        }
    };
    auto pv_mma = [&](int k) __attribute__((always_inline)) {
        const int kb = kbase(k);
        const __bf16* P = Pb + (k & 1) * (HG * kPLd);
        bf16x8 pa[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            pa[mt] = *reinterpret_cast<const bf16x8*>(&P[(16 * mt + l16) * kPLd + 8 * lg]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const i16x4 v0 = lds_read_tr16(Kn + (kb + kvo[nt]));
            const i16x4 v1 = lds_read_tr16(Kn + (kb + kvo[nt]) + 16 * kD);
            const bf16x8 vb = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pa[mt], acc[mt][nt],
                                                                      0, 0, 0);
        }
    };
    auto pv = [&](int k) __attribute__((always_inline)) {
        pv_rescale(k);
        pv_mma(k);
    };

    // QK of tile t (consumer waves): the raw scores, lane holding head hc at
    // rows 4lg + r (first) and 16 + 4lg + r (second).
    struct Scores {
        f32x4 s0, s1;
    };
    auto qk_scores = [&](int t) __attribute__((always_inline)) -> Scores {
        // S^T = K q^T: A operand = K rows (entries), B operand = q (heads).
        // Four accumulator chains (rows 0-15 / 16-31, even / odd k-steps);
        // K fragments are read four k-steps ahead of their MFMAs, one read
        // issued after each MFMA, an order pinned with scheduling-group
        // barriers so LDS latency stays hidden (six k-steps ahead, or pairs
        // of reads after pairs of MFMAs, measured 1-2 % slower).
        const int kb = kbase(t);
        f32x4 sa[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4 sb[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        // Lane (l16, lg) reads rows l16 and 16 + l16 (same swizzle), elements
        // 32ks + 8lg.
        auto kfrag = [&](int rb, int ks) {
            return *reinterpret_cast<const bf16x8*>(Kn + (kb + kq[ks & 7]) + 256 * (ks >> 3) +
                                                    16 * kD * rb);
        };
        constexpr int kAhead = 4;
        bf16x8 fa[kAhead], fb[kAhead];
#pragma unroll
        for (int ks = 0; ks < kAhead; ++ks) {
            fa[ks] = kfrag(0, ks);
            fb[ks] = kfrag(1, ks);
        }
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const bf16x8 qb = __builtin_bit_cast(
                bf16x8, u32x4{rr[4 * ks], rr[4 * ks + 1], rr[4 * ks + 2], rr[4 * ks + 3]});
            sa[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ks % kAhead], qb, sa[ks & 1],
                                                                 0, 0, 0);
            sb[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[ks % kAhead], qb, sb[ks & 1],
                                                                 0, 0, 0);
            if (ks + kAhead < 16) {
                fa[ks % kAhead] = kfrag(0, ks + kAhead);
                fb[ks % kAhead] = kfrag(1, ks + kAhead);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);     // DS reads
#pragma unroll
        for (int ks = 0; ks < 2 * (16 - kAhead); ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);            // DS reads
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * kAhead, 0);
        return Scores{sa[0] + sa[1], sb[0] + sb[1]};
    };

    // Mask + online softmax of tile t (consumer waves), writing P, alpha and
    // the rescale flag of the tile.
    auto softmax = [&](int t, const Scores sc) __attribute__((always_inline)) {
        const f32x4 s0 = sc.s0, s1 = sc.s1;
        const uint32_t vm = vmask[t % kMetaTiles];
        const uint32_t m0 = vm >> (4 * lg), m1 = vm >> (16 + 4 * lg);
        float xs[8];
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            xs[r] = (m0 >> r) & 1u ? s0[r] * p.qk_scale_log2 : -INFINITY;
            xs[4 + r] = (m1 >> r) & 1u ? s1[r] * p.qk_scale_log2 : -INFINITY;
            mx = fmaxf(mx, fmaxf(xs[r], xs[4 + r]));
        }
        mx = xrow_max4(mx);
        // Move the running max only when a score exceeds it by more than the
        // slack (always on the first valid score).
        const bool move = mx > m_run + kRescaleSlack;
        const float m_use = move ? mx : m_run;
        const float a = move ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;   // 0 if m_run = -inf
        // exp2(-inf - m) = 0 for finite m; m_use = -inf only while every
        // score so far is masked, and then every x is -inf too.
        const float m_sub = m_use == -INFINITY ? 0.f : m_use;
        float psum = 0.f;
        bf16x8 pv8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float e = __builtin_amdgcn_exp2f(xs[i] - m_sub);
            psum += e;
            pv8[i] = (__bf16)e;
        }
        l_run = l_run * a + psum;
        m_run = m_use;
        // Slots 8lg .. 8lg+7 of the head's row: entries 4lg + r, then 16 + 4lg + r.
        *reinterpret_cast<bf16x8*>(Pb + (t & 1) * (HG * kPLd) + hc * kPLd + 8 * lg) = pv8;
        if (lg == 0) alpha_s[(t & 1) * HG + hc] = a;
        const bool any = __builtin_amdgcn_ballot_w64(move) != 0;
        if (lane == 0) flags[(t & 1) * 4 + wave] = any ? 1 : 0;
    };

    // Output scale and lse of the consumer lane's head (lanes of row 0).
    const bool direct = p.S == 1;
    auto finish = [&]() __attribute__((always_inline)) {
        const int h = h0 + hc;
        float scale, lse;
        const float M = direct && p.sink ? fmaxf(m_run, sink_l2) : -INFINITY;
        if (M != -INFINITY) {
            // One split with a sink: fold it into the denominator.  M = -inf
            // (no entry and a -inf sink) falls through to the empty case
            // below, since exp2(M - M) would be NaN there.
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
    };

    // Both loops run the same nsteps >= ntiles + 1 steps (a multiple of the
    // producers' unroll, 3 or 6 for dense rows, so their loop body has no
    // branch around a load); steps past ntiles do nothing but the barrier.
    constexpr int kUnroll = DENSE ? 6 : 3;
    const int nsteps = (ntiles + kUnroll) / kUnroll * kUnroll;
    // Pipeline step t = 0..ntiles, then one barrier: QK + softmax of tile t
    // (consumers), PV of tile t-1 (all waves), dequantisation of tile t+1 and
    // loads of tile t+4 (producers), staged resolution of the next half
    // (waves 0..3).  Producers and the other waves run separate loops with
    // the same barriers, so the producers' loop holds no load but their own
    // and the compiler counts them exactly: storing tile t+1 waits for its
    // loads only, with tiles t+2 and t+3 still in flight.
    if (producer && DENSE) {
        // Dense rows take 32 registers a tile, so two tiles are in flight:
        // tile k lives in rr[32(k%2) .. +31]; step t stores tile t+1 into K
        // buffer (t+1)%3 and reuses its registers for tile t+3 (period 6).
        auto dstep = [&](int t, auto kset, auto rset) __attribute__((always_inline)) {
            constexpr int O = 32 * decltype(rset)::value;
            gbyte* a = dense_src(meta_tile(t + 3), prow, t + 3 < ntiles);
            store_dense<O>(rr, prow, l8, Kn + decltype(kset)::value * (kTile * kD));
            load_dense<O>(a, l8, rr);
            if (t >= 1 && t <= ntiles) pv(t - 1);
            __syncthreads();
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        for (int t = 0; t < nsteps; t += 6) {
            dstep(t, I1{}, I1{});
            dstep(t + 1, I2{}, I0{});
            dstep(t + 2, I0{}, I1{});
            dstep(t + 3, I1{}, I0{});
            dstep(t + 4, I2{}, I1{});
            dstep(t + 5, I0{}, I0{});
        }
    } else if (producer) {
        // Tile k's raw bytes live in rr[20(k%3) .. +19]; step t stores tile
        // t+1 into K buffer (t+1)%3 and reuses its registers for tile t+4.
        auto pstep = [&](int t, auto set) __attribute__((always_inline)) {
            constexpr int O = 20 * decltype(set)::value;
            const PatchSrc a = patch_src(meta_tile(t + 4), prow, t + 4 < ntiles);
            store_patch<O, SCRUB>(rr, prow, l8, Kn + decltype(set)::value * (kTile * kD));
            load_patch<O>(a, l8, rr);
            if (t >= 1 && t <= ntiles) pv(t - 1);
            __syncthreads();
        };
        for (int t = 0; t < nsteps; t += 3) {
            pstep(t, std::integral_constant<int, 1>{});
            pstep(t + 1, std::integral_constant<int, 2>{});
            pstep(t + 2, std::integral_constant<int, 0>{});
        }
    } else if (consumer) {
        // Step 0: QK + softmax of tile 0 (or, with no tile, the finish).
        resolve_stage(0);
        if (ntiles > 0)
            softmax(0, qk_scores(0));
        else if (lg == 0)
            finish();
        __syncthreads();
        // Steady state: QK of tile t, then PV of tile t-1 (independent of it)
        // in the same basic block as the softmax of tile t, so the softmax's
        // VALU work overlaps the PV MFMAs.
        for (int t = 1; t < ntiles; ++t) {
            resolve_stage(t);
            pv_rescale(t - 1);
            const Scores sc = qk_scores(t);
            pv_mma(t - 1);
            softmax(t, sc);
            __syncthreads();
        }
        if (ntiles > 0) {
            l_run = xrow_sum4(l_run);
            if (lg == 0) finish();
            pv(ntiles - 1);
            __syncthreads();
        }
        for (int t = ntiles + 1; t < nsteps; ++t) __syncthreads();
    } else {
        for (int t = 0; t < nsteps; ++t) {
            resolve_stage(t);
            if (t >= 1 && t <= ntiles) pv(t - 1);
            __syncthreads();
        }
    }

    // Output (the final bf16 output, or the split's bf16 partial): the
    // scaled accumulators are staged as bf16 rows in LDS, where the K buffers
    // are free after the last step, then written with 16-byte nontemporal
    // stores, one contiguous 1 KB head row per wave instruction.  Written
    // straight from the accumulator layout, each store instruction would
    // scatter 32-byte pieces over 16 rows, and the rows would sit dirty in L2
    // until the end-of-kernel writeback.
    uint16_t* dst;
    int64_t row_stride;
    if (direct) {
        dst = p.out + ((int64_t)b * p.H + h0) * kD;
        row_stride = kD;
    } else {
        dst = p.part_o + (((int64_t)b * p.H + h0) * p.S + s) * kD;
        row_stride = (int64_t)p.S * kD;
    }
    constexpr int kOLd = kD + 8;                 // padded staged row (bf16 elements)
    static_assert(HG * kOLd * 2 <= kKBufs * L::kn_buf, "output staging fits the K buffers");
    static_assert(HG * 64 % kThreads == 0, "whole 16-byte chunks per thread");
    __bf16* Ob = Kn;                             // [HG][kOLd]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const float sc = fin[16 * mt + l16];
        __bf16* row = Ob + (16 * mt + l16) * kOLd + 64 * wave + 4 * lg;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
            bf16x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = (__bf16)(acc[mt][nt][r] * sc);
            *reinterpret_cast<bf16x4*>(row + 16 * nt) = o;
        }
    }
    __syncthreads();
    // 16-byte chunk c of the HG x 1 KB block: head row c / 64, chunk c % 64.
#pragma unroll
    for (int k = 0; k < HG * 64 / kThreads; ++k) {
        const int c = tid + k * kThreads;
        const int h = c >> 6, ch = c & 63;
        const u32x4 v = *reinterpret_cast<const u32x4*>(Ob + h * kOLd + 8 * ch);
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + h * row_stride + 8 * ch));
    }
    // Balanced splits: the token's last split marks the slots it leaves
    // unused as empty (lse -inf), so the combine adds nothing from them.
    // Stored last: stores count on the same counter as loads, so a store
    // ahead of the kernel's loads would hold back every wait on them.
    if (!DENSE && nsplit < p.S && s == nsplit - 1 && tid < HG) {
        float* row = p.part_lse + ((int64_t)b * p.H + h0 + tid) * p.S;
        for (int k = nsplit; k < p.S; ++k) row[k] = -INFINITY;
    }
}

template <int HG, bool SCRUB, bool EMIT = false>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(const DecodeParams p) {
    decode_partial_body<HG, SCRUB, false, EMIT>(p);
}

// Attention over gathered bf16 rows (second kernel of the two-kernel path).
template <int HG>
__global__ __launch_bounds__(kThreads) void dense_partial_kernel(const DecodeParams p) {
    decode_partial_body<HG, false, true>(p);
}

// Two-kernel path, first kernel: gather and dequantise every entry of every
// token's index row into a dense bf16 buffer [B, topk+swa, 512] (row k =
// column k of the index row) with a mask byte per entry (1 = takes no part;
// its row is written as zeros).  (SGLang PR #26208 report, the gather+dequant
// kernel and its output mask.)  32 entries per workgroup, 8 lanes per entry,
// the same row loads and dequantisation as the fused kernel's producers.
template <bool SCRUB>
__global__ __launch_bounds__(kGatherThreads) void gather_dequant_kernel(const DecodeParams p,
                                                                       uint16_t* kv_out,
                                                                       uint8_t* mask_out) {
    const int Kt = p.topk + p.swa;
    const int tiles = (Kt + kTile - 1) / kTile;
    const int b = (int)(blockIdx.x / tiles);
    const int col = (int)(blockIdx.x % tiles) * kTile + (threadIdx.x >> 3);
    const int l8 = threadIdx.x & 7;
    if (col >= Kt) return;                         // no barrier in this kernel
    const int seq = b / p.sq;
    const int vl = p.valid_len ? min(max(p.valid_len[seq], 0), p.topk) : p.topk;
    const int32_t raw = p.idx[(int64_t)b * p.idx_stride + col];
    const int32_t idx = col < p.topk && col >= vl ? -1 : raw;
    const Pool pl = pool_of(p, col >= p.topk);
    const int64_t page = lookup_page(p, pl, seq, idx);
    int64_t m[2];
    write_meta(pl, m, page, idx);
    uint32_t rr[64];
    load_patch<0>(PatchSrc{(gbyte*)m[0], (gbyte*)m[1]}, l8, rr);
    uint16_t* dst = kv_out + ((int64_t)b * Kt + col) * kD;
    const uint64_t sw = (uint64_t)rr[19] << 32 | rr[18];
#pragma unroll
    for (int j = 0; j < 7; ++j) {
        bf16x8 v = dequant8(make_uint2(rr[2 * j], rr[2 * j + 1]), (uint32_t)(sw >> (8 * j)) & 0xFFu);
        if (SCRUB) {
            u32x4 w = __builtin_bit_cast(u32x4, v);
            w = u32x4{scrub_pair(w[0]), scrub_pair(w[1]), scrub_pair(w[2]), scrub_pair(w[3])};
            v = __builtin_bit_cast(bf16x8, w);
        }
        *reinterpret_cast<bf16x8*>(dst + 64 * j + 8 * l8) = v;
    }
#pragma unroll
    for (int j = 7; j < kChunks; ++j) {
        uint2 r = make_uint2(rr[2 * j], rr[2 * j + 1]);
        if (SCRUB) r = make_uint2(scrub_pair(r.x), scrub_pair(r.y));
        *reinterpret_cast<uint2*>(dst + kDNope + 32 * (j - 7) + 4 * l8) = r;
    }
    if (l8 == 0) mask_out[(int64_t)b * Kt + col] = page >= 0 ? 0 : 1;
}

// Merge of split partials with the sink for many (token, head) rows; one
// workgroup per row, 4 output dims per lane.  Splits are taken NB at a time (NB = the split
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
            if (w != 0.f) {                          // an empty split's row is never read into o
                const f32x4 pv = {__uint_as_float(v[j].x << 16), __uint_as_float(v[j].x & 0xFFFF0000u),
                                  __uint_as_float(v[j].y << 16), __uint_as_float(v[j].y & 0xFFFF0000u)};
                o += w * pv;
            }
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

// Merge of split partials for few (token, head) rows: the row's 512 dims
// are cut into Q slices of 512/Q dims, one workgroup of W waves per slice,
// each lane holding 512/(64 Q) dims.  Wave w merges splits w, w + W, ...
// (at most NSW of them; S <= 64).  Every wave loads the row's S lse values,
// one per lane, with its partial loads (one memory round trip), and reduces
// them to the common maximum M (sink included) and the weights
// e^(lse_s - M); the waves' weighted sums then share one scale and are added
// in LDS in wave order, so the result is deterministic for a given S.  A
// split of weight 0 (empty, lse = -inf) adds nothing, whatever its partial
// holds.
template <int Q, int W, int NSW>
__global__ __launch_bounds__(64 * W) void combine_slice_kernel(const CombineParams p) {
    constexpr int DPL = kD / (Q * 64);           // dims per lane
    constexpr int WPL = DPL / 2;                 // bf16 pairs per lane
    static_assert(WPL == 1 || WPL == 2 || WPL == 4, "slice width");
    static_assert(W * NSW <= 64, "splits beyond one lse per lane");
    __shared__ float part[W > 1 ? W - 1 : 1][DPL][64];
    const int64_t bh = blockIdx.x / Q;
    const int qd = (int)(blockIdx.x % Q);
    const int h = (int)(bh % p.H);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int S = p.S;
    const float lraw = p.part_lse[bh * S + min(lane, S - 1)];
    const uint32_t* po = reinterpret_cast<const uint32_t*>(p.part_o + bh * S * kD + qd * (kD / Q)) +
                         lane * WPL;
    // Unconditional loads: splits past S re-read split S - 1 and get weight 0.
    uint32_t v[NSW][WPL];
#pragma unroll
    for (int j = 0; j < NSW; ++j) {
        const uint32_t* src = po + (int64_t)min(wave + W * j, S - 1) * (kD / 2);
        if constexpr (WPL == 1) {
            v[j][0] = src[0];
        } else if constexpr (WPL == 2) {
            const uint2 t = *reinterpret_cast<const uint2*>(src);
            v[j][0] = t.x;
            v[j][1] = t.y;
        } else {
            const uint4 t = *reinterpret_cast<const uint4*>(src);
            v[j][0] = t.x;
            v[j][1] = t.y;
            v[j][2] = t.z;
            v[j][3] = t.w;
        }
    }
    const float sink = p.sink ? p.sink[h] : -INFINITY;
    const float lv = lane < S ? lraw : -INFINITY;
    const float M = fmaxf(xrow_max4(row_max16(lv)), sink);
    const bool live = M != -INFINITY;
    const float wl = (live && lv != -INFINITY) ? __builtin_amdgcn_exp2f((lv - M) * kLog2e) : 0.f;
    float o[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) o[d] = 0.f;
#pragma unroll
    for (int j = 0; j < NSW; ++j) {
        const float w = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), wave + W * j));
        if (w != 0.f) {
#pragma unroll
            for (int k = 0; k < WPL; ++k) {
                o[2 * k] += w * __uint_as_float(v[j][k] << 16);
                o[2 * k + 1] += w * __uint_as_float(v[j][k] & 0xFFFF0000u);
            }
        }
    }
    if constexpr (W > 1) {
        if (wave > 0) {
#pragma unroll
            for (int d = 0; d < DPL; ++d) part[wave - 1][d][lane] = o[d];
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int k = 0; k < W - 1; ++k)
#pragma unroll
            for (int d = 0; d < DPL; ++d) o[d] += part[k][d][lane];
    }
    float D = xrow_sum4(row_sum16(wl));
    if (live && sink != -INFINITY) D += __builtin_amdgcn_exp2f((sink - M) * kLog2e);
    const float inv = live ? 1.f / D : 0.f;
    uint32_t pk[WPL];
#pragma unroll
    for (int k = 0; k < WPL; ++k)
        pk[k] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(o[2 * k] * inv)) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(o[2 * k + 1] * inv)) << 16);
    uint32_t* dst = reinterpret_cast<uint32_t*>(p.out + bh * kD + qd * (kD / Q)) + lane * WPL;
    if constexpr (WPL == 1)
        dst[0] = pk[0];
    else if constexpr (WPL == 2)
        *reinterpret_cast<uint2*>(dst) = make_uint2(pk[0], pk[1]);
    else
        *reinterpret_cast<uint4*>(dst) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    if (qd == 0 && lane == 0 && p.lse)
        p.lse[bh] = live ? M + __builtin_amdgcn_logf(D) * kLn2 : -INFINITY;
}

// Gather floor: the partial kernel's work units (same grid, same XCD
// mapping, same per-split entry range) and the same row loads (8 lanes per
// row, 9 x 8 data bytes + the 8-byte scale word, rows that take no part read
// the zero row), with no LDS tile and no arithmetic beyond folding the loaded
// words into one word per thread.  Resolution of up to 1024 entries goes to
// LDS first; the loads then run 4 passes of 64 rows deep.  Its duration is
// the floor the partial kernel's memory traffic sets.
__global__ __launch_bounds__(kThreads) void gather_floor_kernel(const DecodeParams p,
                                                                uint32_t* words) {
    __shared__ int64_t addr[kMetaTiles * kTile][2];
    const int64_t Lb = blockIdx.x;
    const int x = (int)(Lb % kXcds);
    const int64_t r8 = Lb / kXcds;
    const int64_t unit = (r8 / p.G) * kXcds + x;
    if (unit >= p.units) return;
    const int b = (int)(unit / p.S);
    const int s = (int)(unit % p.S);
    const int seq = b / p.sq;
    const int vl = p.valid_len ? min(max(p.valid_len[seq], 0), p.topk) : p.topk;
    const int eff = vl + p.swa;
    int chunk = (eff + p.S - 1) / p.S;
    chunk = (chunk + kTile - 1) / kTile * kTile;
    const int lo = min(s * chunk, eff);
    const int hi = min(lo + chunk, eff);
    const int tid = threadIdx.x, row = tid >> 3, l8 = tid & 7;
    constexpr int kRing = kMetaTiles * kTile;            // 1024 entries
    uint32_t acc = 0;
    for (int base = lo; base < hi; base += kRing) {
        // Two entries a thread: both index loads, then both table loads, in
        // flight together (two round trips, as in the partial kernel).
        int32_t id[2], w[2] = {0, 0};
        Pool pl[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            id[e] = load_index(p, b, vl, hi, base + tid + e * kThreads);
            pl[e] = pool_of(p, base + tid + e * kThreads >= vl);
        }
        if (p.bt) {
#pragma unroll
            for (int e = 0; e < 2; ++e)
                w[e] = pl[e].bt[(int64_t)seq * pl[e].bt_stride + table_column(pl[e], id[e])];
        }
#pragma unroll
        for (int e = 0; e < 2; ++e)
            write_meta(pl[e], addr[tid + e * kThreads], page_from_word(p, pl[e], id[e], w[e]),
                       id[e]);
        __syncthreads();
        const int n = min(hi - base, kRing);
        for (int r0 = 0; r0 < n; r0 += 4 * 64) {
            uint64_t v[4][kChunks + 1];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int r = r0 + 64 * h + row;
                gbyte* src = (gbyte*)(r < n ? addr[r][0] : reinterpret_cast<int64_t>(kZeroRow));
                gbyte* sc = (gbyte*)(r < n ? addr[r][1] : reinterpret_cast<int64_t>(kZeroRow));
#pragma unroll
                for (int j = 0; j < kChunks; ++j) v[h][j] = *(gu64*)(src + 8 * l8 + 64 * j);
                v[h][kChunks] = *(gu64*)sc;
            }
            // The scale word is loaded by all 8 lanes of a row and folded by one.
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                if (l8 != 0) v[h][kChunks] = 0;
#pragma unroll
                for (int j = 0; j <= kChunks; ++j) acc ^= (uint32_t)v[h][j] ^ (uint32_t)(v[h][j] >> 32);
            }
        }
        __syncthreads();
    }
    words[Lb * kThreads + tid] = acc;
}

hipError_t launch_gather_floor(const DecodeParams& p, int64_t grid, uint32_t* words,
                               hipStream_t stream) {
    hipLaunchKernelGGL(gather_floor_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p,
                       words);
    return hipGetLastError();
}

template <bool SCRUB>
static hipError_t launch_partial_variant(const DecodeParams& p, int heads_per_group,
                                         dim3 g, hipStream_t stream) {
    const dim3 blk(kThreads);
    if (p.slots) {
        switch (heads_per_group) {
            case 16: hipLaunchKernelGGL((decode_partial_kernel<16, SCRUB, true>), g, blk, 0, stream, p); break;
            case 32: hipLaunchKernelGGL((decode_partial_kernel<32, SCRUB, true>), g, blk, 0, stream, p); break;
            case 48: hipLaunchKernelGGL((decode_partial_kernel<48, SCRUB, true>), g, blk, 0, stream, p); break;
            case 64: hipLaunchKernelGGL((decode_partial_kernel<64, SCRUB, true>), g, blk, 0, stream, p); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    switch (heads_per_group) {
        case 16: hipLaunchKernelGGL((decode_partial_kernel<16, SCRUB>), g, blk, 0, stream, p); break;
        case 32: hipLaunchKernelGGL((decode_partial_kernel<32, SCRUB>), g, blk, 0, stream, p); break;
        case 48: hipLaunchKernelGGL((decode_partial_kernel<48, SCRUB>), g, blk, 0, stream, p); break;
        case 64: hipLaunchKernelGGL((decode_partial_kernel<64, SCRUB>), g, blk, 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_dense_partial(const DecodeParams& p, int heads_per_group, int64_t grid,
                                hipStream_t stream) {
    const dim3 g((unsigned)grid), blk(kThreads);
    switch (heads_per_group) {
        case 16: hipLaunchKernelGGL(dense_partial_kernel<16>, g, blk, 0, stream, p); break;
        case 32: hipLaunchKernelGGL(dense_partial_kernel<32>, g, blk, 0, stream, p); break;
        case 48: hipLaunchKernelGGL(dense_partial_kernel<48>, g, blk, 0, stream, p); break;
        case 64: hipLaunchKernelGGL(dense_partial_kernel<64>, g, blk, 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gather_dequant(const DecodeParams& p, uint16_t* kv_out, uint8_t* mask_out,
                                 bool scrub, hipStream_t stream) {
    const int64_t grid = (int64_t)p.B * ((p.topk + p.swa + kTile - 1) / kTile);
    if (scrub)
        hipLaunchKernelGGL(gather_dequant_kernel<true>, dim3((unsigned)grid), dim3(kGatherThreads),
                           0, stream, p, kv_out, mask_out);
    else
        hipLaunchKernelGGL(gather_dequant_kernel<false>, dim3((unsigned)grid), dim3(kGatherThreads),
                           0, stream, p, kv_out, mask_out);
    return hipGetLastError();
}

hipError_t launch_decode_partial(const DecodeParams& p, int heads_per_group, int64_t grid,
                                 bool scrub, hipStream_t stream) {
    // The conversion output needs the block table, a single pool and at most
    // 1024 columns per split.
    if (p.slots != nullptr && (p.bt == nullptr || p.kv2 != nullptr || p.bal != 0 ||
                               (p.topk + p.swa + p.S - 1) / p.S > 2 * kThreads))
        return hipErrorInvalidValue;
    // Balanced splits: the batch's tokens fit one wave's lanes.
    if (p.bal != 0 && (p.B > 64 || p.S < 2 || p.units != (int64_t)p.B * p.bal))
        return hipErrorInvalidValue;
    const dim3 g((unsigned)grid);
    return scrub ? launch_partial_variant<true>(p, heads_per_group, g, stream)
                 : launch_partial_variant<false>(p, heads_per_group, g, stream);
}

template <int Q, int W>
static void launch_combine_slices(const CombineParams& p, dim3 g, dim3 blk, hipStream_t stream) {
    const int nsw = (p.S + W - 1) / W;
    if (nsw <= 2)
        hipLaunchKernelGGL((combine_slice_kernel<Q, W, 2>), g, blk, 0, stream, p);
    else if (nsw <= 4)
        hipLaunchKernelGGL((combine_slice_kernel<Q, W, 4>), g, blk, 0, stream, p);
    else if (nsw <= 8)
        hipLaunchKernelGGL((combine_slice_kernel<Q, W, 8>), g, blk, 0, stream, p);
    else if (nsw <= 16)
        hipLaunchKernelGGL((combine_slice_kernel<Q, W, 16>), g, blk, 0, stream, p);
    else
        hipLaunchKernelGGL((combine_slice_kernel<Q, W, 64 / W>), g, blk, 0, stream, p);
}

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
    const CombineShape cs = combine_shape((int64_t)p.B * p.H, p.S);
    const dim3 g((unsigned)cs.grid), blk((unsigned)cs.block);
    if (cs.slices == 4 && cs.waves == 4) {
        launch_combine_slices<4, 4>(p, g, blk, stream);
        return hipGetLastError();
    }
    if (cs.slices == 2 && cs.waves == 2) {
        launch_combine_slices<2, 2>(p, g, blk, stream);
        return hipGetLastError();
    }
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
