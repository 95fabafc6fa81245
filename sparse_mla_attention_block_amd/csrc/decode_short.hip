// Short-split decode kernel for gfx950: one workgroup per (token, split,
// head group) whose split holds at most 128 entries (two super-tiles of 64
// cache rows).  It is the latency-bound regime of long-context decode at low
// batch (vLLM PR #52212 page, motivation: the old split-K path lacked
// parallelism there; implementation item 2: many splits per row): each
// workgroup sees only one or two tiles, so instead of a software pipeline
// every phase of a super-tile runs on all 8 waves at once:
//   1. every lane resolves one cache row per super-tile itself (index ->
//      page through the block table -> row address; 8 lanes per row) and
//      issues that row's loads, for both super-tiles up front, while the QK
//      waves load q; the rows of super-tile 0 are dequantised into the LDS
//      K tile (FP8 x 2^(code-127) -> bf16, the gfx950 scaled convert);
//   2. QK on bf16 MFMA 16x16x32 (S^T = K q^T), the (16-row block, 16-head
//      block) pairs spread over the 8 waves (with 16 heads, the 512-dim dot
//      is cut into two halves instead), scores to LDS;
//   3. mask + softmax: 8 or 16 lanes per head, each holding 4 or 8 scores,
//      wave reductions over DPP rows; online across the two super-tiles;
//      bf16 probabilities to LDS in the MFMA's k order;
//   4. PV on bf16 MFMA, wave w owning output dims [64w, 64w+64), V read from
//      the K tile through the LDS transpose read.
// Four barriers per super-tile, no other synchronisation.  The epilogue is
// the pipelined kernel's: with one split the sink is folded in and bf16
// output and lse are written, with several the split's normalised bf16
// partial and its lse.  Rows that take no part read the zero row, so a NaN
// in the cache never reaches an MFMA.
//
// Each workgroup runs this code once, and every launch starts with a cold
// instruction cache, so the bytes of code a workgroup executes cost about as
// much time as its memory round trips (measured on MI355X: about one cycle
// per byte).  The kernel is therefore written for a short instruction
// stream: 32-bit index arithmetic with launch-time divisors, a K tile with a
// padded row stride so that every LDS access is a base address plus an
// immediate offset, the block-table lookup chosen at compile time, and loads
// that sit outside every branch, so that the compiler can wait for exactly
// the loads a step needs.  Dual-pool decodes use the pipelined kernel.
#include <hip/hip_runtime.h>
#include <math.h>

#include "decode_common.hpp"
#include "device_util.hpp"
#include "internal.hpp"

namespace dsv4 {

template <int HG>
struct ShortSmem {
    static constexpr int MT = HG / 16;
    static constexpr int NS = MT == 1 ? 2 : 1;                   // score planes (k halves)
    static constexpr int sc_ld = kShortRows + 4;                  // f32 per score row
    static constexpr int pb_ld = kShortRows + 8;                  // bf16 per probability row
    static constexpr int kn = 0;                                  // [64][520] bf16
    static constexpr int sc = kn + kShortRows * kShortLd * 2;     // [NS][HG][sc_ld] f32
    static constexpr int pb = sc + NS * HG * sc_ld * 4;           // [HG][pb_ld] bf16
    static constexpr int alpha = pb + HG * pb_ld * 2;             // [HG] f32
    static constexpr int fin = alpha + HG * 4;                    // [HG] f32
    static constexpr int valid = fin + HG * 4;                    // [2][64] u8
    static constexpr int bytes = valid + kShortMaxSuper * kShortRows;
    static_assert(sc % 16 == 0 && pb % 16 == 0 && valid % 16 == 0, "alignment");
    static_assert(bytes <= 160 * 1024, "LDS");
};

size_t short_lds_bytes(int hg) {
    return hg == 16 ? ShortSmem<16>::bytes : hg == 32 ? ShortSmem<32>::bytes : ShortSmem<64>::bytes;
}

// STAMPS: thread 0 of each workgroup records its phase timeline into
// p.timeline (a measurement variant; see dsv4_short_timeline).
// EMIT (with TABLE): the workgroups of head group 0 also write the req-local
// -> global conversion of the token's index row into p.slots (vLLM PR #41217
// report, key source snippets: the conversion kernel), split s taking
// columns [s*cc, s*cc + cc) with cc = ceil((topk + swa) / S) <= 128, one per
// lane; its index and table loads ride in the decode's own round trips.
// ONE: every split holds at most one super-tile (kShortRows entries); the
// second super-tile's index, table and row loads, its dequantisation and
// the online rescale between super-tiles are left out.  A quarter less code
// (4.0 against 5.2 KB for 16 heads writing the slots), and the code a
// workgroup runs once from a cold instruction cache is its largest cost.
template <int HG, bool SCRUB, bool TABLE, bool STAMPS = false, bool EMIT = false, bool ONE = false>
__global__ __launch_bounds__(kThreads) void decode_short_kernel(const DecodeParams p) {
    constexpr int MT = HG / 16;
    static_assert(MT == 1 || MT == 2 || MT == 4, "short kernel head groups: 16, 32, 64");
    static_assert(!EMIT || (TABLE && !STAMPS), "the conversion output needs the block table");
    using L = ShortSmem<HG>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[L::bytes];
    __bf16* Kt = reinterpret_cast<__bf16*>(smem + L::kn);
    float* Sc = reinterpret_cast<float*>(smem + L::sc);
    __bf16* Pb = reinterpret_cast<__bf16*>(smem + L::pb);
    float* alpha_s = reinterpret_cast<float*>(smem + L::alpha);
    float* fin = reinterpret_cast<float*>(smem + L::fin);
    uint8_t* vflag = smem + L::valid;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    // Stamps stay in scalar registers and are stored once, at the end, so
    // that recording them changes the instruction stream as little as it can.
    uint64_t ts[kTimelineStamps] = {};
    auto mark = [&](int k, bool real) __attribute__((always_inline)) {
        if constexpr (STAMPS)
            ts[k] = real ? __builtin_amdgcn_s_memrealtime() : __builtin_amdgcn_s_memtime();
    };
    // Every kernel argument the kernel reads, in one batch of scalar loads
    // and one wait: otherwise the compiler loads them in three batches, each
    // after a branch that depends on the one before.
    asm volatile("" ::"s"(p.q), "s"(p.kv), "s"(p.bt), "s"(p.idx), "s"(p.valid_len),
                 "s"(p.sink), "s"(p.out), "s"(p.lse), "s"(p.part_o), "s"(p.part_lse),
                 "s"(p.num_blocks), "s"(p.bt_stride), "s"(p.page_stride), "s"(p.idx_stride),
                 "s"(p.units), "s"(p.H), "s"(p.topk), "s"(p.swa), "s"(p.max_blocks), "s"(p.S),
                 "s"(p.G), "s"(p.qk_scale_log2), "s"(p.slots), "s"(p.timeline));
    asm volatile("" ::"s"(p.fd_S.d), "s"(p.fd_S.m), "s"(p.fd_S.l), "s"(p.fd_G.m), "s"(p.fd_G.l),
                 "s"(p.fd_sq.m), "s"(p.fd_sq.l), "s"(p.fd_bs.d), "s"(p.fd_bs.m), "s"(p.fd_bs.l));
    mark(0, true);
    mark(1, false);

    // Work unit: the pipelined kernel's mapping (head groups of one split
    // kXcds apart, on one XCD), in 32-bit arithmetic.
    const uint32_t Lb = blockIdx.x;
    const uint32_t r8 = Lb / kXcds;
    const uint32_t gq = fdiv(r8, p.fd_G);
    const uint32_t g = r8 - gq * (uint32_t)p.G;
    const uint32_t unit = gq * kXcds + Lb % kXcds;
    if (unit >= (uint64_t)p.units) return;
    const uint32_t b = fdiv(unit, p.fd_S);
    const uint32_t s = unit - b * (uint32_t)p.S;
    const uint32_t seq = fdiv(b, p.fd_sq);
    const int h0 = (int)g * HG;

    const int vl = p.valid_len ? min(max(p.valid_len[seq], 0), p.topk) : p.topk;
    const int eff = vl + p.swa;
    const int chunk = (int)(fdiv((uint32_t)(eff + p.S - 1), p.fd_S) + kTile - 1) / kTile * kTile;
    const int lo = min((int)s * chunk, eff);
    const int hi = min(lo + chunk, eff);
    const int n = hi - lo;                                   // <= 128 (the plan's bound)

    // 1. Resolution and row loads: lane (prow, l8) serves row prow of each
    // super-tile.  Index loads first, then q, then the block-table loads,
    // then the rows; every load is unconditional.
    const int prow = 8 * wave + (lane >> 4) + 4 * ((lane >> 3) & 1), l8 = lane & 7;
    const int e0 = lo + prow, e1 = e0 + kShortRows;
    const int32_t* irow = p.idx + (int64_t)b * p.idx_stride;
    auto index_at = [&](int pos) -> int32_t {
        const bool in = pos < hi;
        const int col = pos < vl ? pos : p.topk + (pos - vl);
        const int32_t v = *global(irow + (in ? col : 0));
        return in ? v : -1;
    };
    const int32_t i0 = index_at(e0);
    const int32_t i1 = ONE ? -1 : index_at(e1);
    // Conversion column of this lane (EMIT).
    const uint32_t kt = (uint32_t)(p.topk + p.swa);
    int cv_col = 0;
    bool cv_on = false;
    int32_t cv_idx = -1;
    if constexpr (EMIT) {
        const uint32_t cc = fdiv(kt + (uint32_t)p.S - 1, p.fd_S);
        cv_col = (int)(s * cc) + tid;
        cv_on = g == 0 && tid < (int)cc && (uint32_t)cv_col < kt;
        const int32_t v = *global(irow + (cv_on ? cv_col : 0));
        cv_idx = cv_on ? v : -1;
    }

    // QK assignment: 16 heads cut the dot into two k halves (wave w: row
    // block w&3, half w>>2); 32 heads give each wave one (row block, head
    // block) pair; 64 heads two row blocks of one head block.
    constexpr int KSTEPS = MT == 1 ? 8 : 16;
    constexpr int NRB = MT == 4 ? 2 : 1;
    const int qk_hb = MT == 1 ? 0 : MT == 2 ? (wave >> 2) : (wave & 3);
    const int qk_rb0 = MT == 4 ? 2 * (wave >> 2) : (wave & 3);
    const int qk_k0 = MT == 1 ? KSTEPS * (wave >> 2) : 0;
    uint32_t qr[4 * KSTEPS];
    {
        const u32x4* qp = reinterpret_cast<const u32x4*>(
            p.q + ((int64_t)b * p.H + h0 + 16 * qk_hb + l16) * kD + 32 * qk_k0 + 8 * lg);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const u32x4 v = qp[4 * ks];
            qr[4 * ks] = v[0];
            qr[4 * ks + 1] = v[1];
            qr[4 * ks + 2] = v[2];
            qr[4 * ks + 3] = v[3];
        }
    }

    // Softmax lanes: TPH lanes per head, EPT entries each.
    constexpr int TPH = (kThreads / HG) < 16 ? (kThreads / HG) : 16;
    constexpr int EPT = kShortRows / TPH;
    const int sm_h = tid / TPH, sm_j = tid % TPH;
    const bool sm_active = tid < HG * TPH;
    // The sink is loaded unconditionally here and used in the epilogue.
    const float sink_raw = *global(p.sink ? p.sink + h0 + (sm_active ? sm_h : 0) : &kZeroFloat);

    // Table words, then the rows of both super-tiles (of the one, with ONE;
    // zero rows past the split's end), all unconditional.
    const int32_t w0 = table_word<TABLE>(p, seq, i0);
    const int32_t w1 = ONE ? 0 : table_word<TABLE>(p, seq, i1);
    int32_t cv_word = 0;
    if constexpr (EMIT) cv_word = table_word<true>(p, seq, cv_idx);
    uint32_t rr[64];
    bool live0, live1 = false;
    load_patch<0>(row_source<TABLE>(p, i0, w0, live0), l8, rr);
    if constexpr (!ONE) load_patch<20>(row_source<TABLE>(p, i1, w1, live1), l8, rr);
    if (l8 == 0) {
        vflag[prow] = live0 ? 1 : 0;
        if constexpr (!ONE) vflag[kShortRows + prow] = live1 ? 1 : 0;
    }
    mark(2, false);
    store_row<0, SCRUB>(rr, prow, l8, Kt);
    mark(3, false);
    if constexpr (EMIT) {
        // The conversion's rule: a negative index, a block past the table, a
        // negative page entry or a slot past INT32_MAX give the fill -1.
        if (cv_on) {
            const uint32_t ui = cv_idx >= 0 ? (uint32_t)cv_idx : 0u;
            const uint32_t blk = fdiv(ui, p.fd_bs);
            const int64_t gs = (int64_t)cv_word * p.fd_bs.d + (ui - blk * p.fd_bs.d);
            const bool ok = cv_idx >= 0 && blk < (uint32_t)p.max_blocks && cv_word >= 0 &&
                            gs <= (int64_t)INT32_MAX;
            p.slots[(int64_t)b * kt + cv_col] = ok ? (int32_t)gs : -1;
        }
    }
    __syncthreads();
    mark(4, false);

    // Online-softmax state of a softmax lane's head (replicated over its TPH
    // lanes), base-2 units.
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nst = ONE ? 1 : (n + kShortRows - 1) / kShortRows;
    for (int st = 0; st < nst; ++st) {
        const int nrows = min(n - st * kShortRows, kShortRows);   // rows that may take part

        // 2. QK: scores of the wave's row block(s) for its head block.
#pragma unroll
        for (int j = 0; j < NRB; ++j) {
            const int rb = qk_rb0 + j;
            if (16 * rb < nrows) {
                f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
                const __bf16* krow = Kt + (16 * rb + l16) * kShortLd + 32 * qk_k0 + 8 * lg;
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 32 * ks);
                    const bf16x8 qb = __builtin_bit_cast(
                        bf16x8, u32x4{qr[4 * ks], qr[4 * ks + 1], qr[4 * ks + 2], qr[4 * ks + 3]});
                    if (ks & 1)
                        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qb, c1, 0, 0, 0);
                    else
                        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qb, c0, 0, 0, 0);
                }
                // Lane (l16, lg) holds head 16*hb + l16 at rows 16rb + 4lg + r.
                const int plane = MT == 1 ? (wave >> 2) : 0;
                *reinterpret_cast<f32x4*>(
                    Sc + (plane * HG + 16 * qk_hb + l16) * L::sc_ld + 16 * rb + 4 * lg) = c0 + c1;
            }
        }
        __syncthreads();
        if (st == 0) mark(5, false);

        // 3. Mask + online softmax of the super-tile.
        if (sm_active) {
            const int e = sm_j * EPT;
            const float* sr = Sc + sm_h * L::sc_ld + e;
            const uint8_t* vf = vflag + st * kShortRows + e;
            float xs[EPT];
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < EPT; ++i) {
                float v = sr[i];
                if constexpr (MT == 1) v += sr[HG * L::sc_ld + i];
                xs[i] = vf[i] ? v * p.qk_scale_log2 : -INFINITY;
                mx = fmaxf(mx, xs[i]);
            }
            mx = group_max<TPH>(mx);
            const float m_new = fmaxf(m_run, mx);
            const float m_sub = m_new == -INFINITY ? 0.f : m_new;
            const float a = __builtin_amdgcn_exp2f(m_run - m_sub);   // 0 while nothing was seen
            float ps = 0.f;
            typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
#pragma unroll
            for (int q4 = 0; q4 < EPT / 4; ++q4) {
                bf16x4 pv4;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pe = __builtin_amdgcn_exp2f(xs[4 * q4 + i] - m_sub);
                    ps += pe;
                    pv4[i] = (__bf16)pe;
                }
                *reinterpret_cast<bf16x4*>(Pb + sm_h * L::pb_ld + k_slot(e + 4 * q4)) = pv4;
            }
            ps = group_sum<TPH>(ps);
            l_run = ONE ? ps : l_run * a + ps;
            m_run = m_new;
            if (!ONE && sm_j == 0) alpha_s[sm_h] = a;
        }
        __syncthreads();
        if (st == 0) mark(6, false);

        // 4. PV: O^T += V^T P^T over the super-tile's k-steps.
        if constexpr (!ONE) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float a = alpha_s[16 * mt + l16];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) acc[mt][nt] *= a;
            }
        }
        const __bf16* vbase = Kt + (4 * lg + (l16 >> 2)) * kShortLd + 64 * wave + 4 * (l16 & 3);
        const __bf16* pbase = Pb + l16 * L::pb_ld + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (32 * ks < nrows) {
                bf16x8 pa[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    pa[mt] = *reinterpret_cast<const bf16x8*>(pbase + 16 * mt * L::pb_ld + 32 * ks);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const __bf16* vp = vbase + 32 * ks * kShortLd + 16 * nt;
                    const i16x4 v0 = lds_read_tr16(vp);
                    const i16x4 v1 = lds_read_tr16(vp + 16 * kShortLd);
                    const bf16x8 vb = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[mt][nt] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pa[mt], acc[mt][nt], 0, 0, 0);
                }
            }
        }
        if (st + 1 < nst) {
            __syncthreads();                           // K tile and P free again
            store_row<20, SCRUB>(rr, prow, l8, Kt);
            __syncthreads();
        }
    }

    mark(7, false);
    // Epilogue: output scale and lse per head (one softmax lane per head).
    const bool direct = p.S == 1;
    if (sm_active && sm_j == 0) {
        const int h = h0 + sm_h;
        const float sink_l2 = p.sink ? sink_raw * kLog2e : -INFINITY;
        float scale, lse;
        const float M = direct && p.sink ? fmaxf(m_run, sink_l2) : -INFINITY;
        if (M != -INFINITY) {
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
        fin[sm_h] = scale;
        if (direct) {
            if (p.lse) p.lse[(int64_t)b * p.H + h] = lse;
        } else {
            p.part_lse[((int64_t)b * p.H + h) * p.S + s] = lse;
        }
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
    // The scaled accumulators are staged as bf16 rows in the (now free) K
    // tile, then written with 16-byte stores, one contiguous 1 KB head row per
    // wave instruction: nontemporal for the final output, ordinary for the
    // split partials, which the combine reads right after (ordinary stores
    // made the two-launch step 3 % faster; the pipelined kernel's larger
    // partials measured the other way).
    static_assert(HG <= kShortRows && HG * 64 % kThreads == 0, "output staging");
    __bf16* obase = Kt + l16 * kShortLd + 64 * wave + 4 * lg;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const float sc = fin[16 * mt + l16];
        __bf16* orow = obase + 16 * mt * kShortLd;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
            bf16x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = (__bf16)(acc[mt][nt][r] * sc);
            *reinterpret_cast<bf16x4*>(orow + 16 * nt) = o;
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < HG * 64 / kThreads; ++k) {
        const int c = tid + k * kThreads;
        const int h = c >> 6, ch = c & 63;
        const u32x4 v = *reinterpret_cast<const u32x4*>(Kt + h * kShortLd + 8 * ch);
        u32x4* o = reinterpret_cast<u32x4*>(dst + h * row_stride + 8 * ch);
        if (direct)
            __builtin_nontemporal_store(v, o);
        else
            *o = v;
    }
    if constexpr (STAMPS) {
        mark(8, false);
        mark(9, true);
        if (tid == 0) {
            uint64_t* stamp = p.timeline + (size_t)blockIdx.x * kTimelineStamps;
#pragma unroll
            for (int k = 0; k < kTimelineStamps; ++k) stamp[k] = ts[k];
        }
    }
}

template <int HG, bool ONE>
static void launch_short_hg(const DecodeParams& p, dim3 g, bool scrub, hipStream_t stream) {
    const dim3 blk(kThreads);
    const bool table = p.bt != nullptr;
    if (p.timeline) {
        if (table)
            hipLaunchKernelGGL((decode_short_kernel<HG, false, true, true, false, ONE>), g, blk, 0,
                               stream, p);
        else
            hipLaunchKernelGGL((decode_short_kernel<HG, false, false, true, false, ONE>), g, blk,
                               0, stream, p);
        return;
    }
    if (p.slots) {
        if (scrub)
            hipLaunchKernelGGL((decode_short_kernel<HG, true, true, false, true, ONE>), g, blk, 0,
                               stream, p);
        else
            hipLaunchKernelGGL((decode_short_kernel<HG, false, true, false, true, ONE>), g, blk, 0,
                               stream, p);
        return;
    }
    if (scrub) {
        if (table)
            hipLaunchKernelGGL((decode_short_kernel<HG, true, true, false, false, ONE>), g, blk, 0,
                               stream, p);
        else
            hipLaunchKernelGGL((decode_short_kernel<HG, true, false, false, false, ONE>), g, blk,
                               0, stream, p);
    } else {
        if (table)
            hipLaunchKernelGGL((decode_short_kernel<HG, false, true, false, false, ONE>), g, blk,
                               0, stream, p);
        else
            hipLaunchKernelGGL((decode_short_kernel<HG, false, false, false, false, ONE>), g, blk,
                               0, stream, p);
    }
}

hipError_t launch_decode_short(const DecodeParams& p, int heads_per_group, int64_t grid,
                               bool scrub, hipStream_t stream) {
    if (p.kv2 != nullptr) return hipErrorInvalidValue;     // single pool only
    if (p.slots != nullptr && (p.bt == nullptr || p.timeline != nullptr))
        return hipErrorInvalidValue;
    const dim3 g((unsigned)grid);
    // Splits of at most one super-tile (every split's chunk, whole tiles, at
    // most kShortRows entries) run the variant without the second one.
    const int64_t kt = (int64_t)p.topk + p.swa;
    const bool one = ((kt + p.S - 1) / p.S + kTile - 1) / kTile * kTile <= kShortRows;
    switch (heads_per_group) {
        case 16: one ? launch_short_hg<16, true>(p, g, scrub, stream)
                     : launch_short_hg<16, false>(p, g, scrub, stream); break;
        case 32: one ? launch_short_hg<32, true>(p, g, scrub, stream)
                     : launch_short_hg<32, false>(p, g, scrub, stream); break;
        case 64: one ? launch_short_hg<64, true>(p, g, scrub, stream)
                     : launch_short_hg<64, false>(p, g, scrub, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dsv4
