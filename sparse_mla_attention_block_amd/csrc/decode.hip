// Sparse FP8 MLA decode kernels for gfx950 (CDNA4): the partial (split-K)
// kernel and the log-sum-exp combine kernel.
//
// Method sources (page titles):
//   vLLM PR #52212, gfx950 DSV4 sparse decode page, implementation item 1:
//     one 512-wide QK dot over 448 NoPE + 64 RoPE dims, PV in 4 slabs of 128
//     dims, 32-row guarded tiles, masked tail, attention sink and invalid
//     indices; item 2: split-K with per-row active splits.
//   SGLang PR #26208 report, key source snippets: fp8_ds_mla row and page
//     layout, -1 invalid marker, top-k length mask; review highlights: a
//     masked or -inf score contributes exactly zero to the running sum.
//
// One workgroup = 4 waves = 256 lanes serves one (token b, split s, head
// group g).  Per tile of 32 cache rows:
//   1. lanes 0..31 resolve their entry's page and byte offsets (int64);
//   2. every lane gathers an 8-row x 8-dim patch (8-byte loads, coalesced in
//      128-byte runs per row), dequantises FP8 x 2^(code-127) to bf16 and
//      stores it twice in LDS: row-major (K operand of QK) and transposed
//      (V operand of PV), so both MFMA operands are 16-byte LDS reads;
//      rows that do not take part are stored as zeros, so no NaN in the
//      cache can reach an MFMA;
//   3. QK on bf16 MFMA 16x16x32 with q held in registers, scores scaled to
//      base 2 and masked to -inf;
//   4. online softmax (one head per 4 lanes, 8 scores each, butterfly
//      reductions); the running sum takes the fp32 probabilities, the PV
//      operand their bf16 rounding;
//   5. PV on bf16 MFMA: wave w owns output dims [128w, 128w+128) for every
//      head of the group (the 4 x 128 accumulator slabs), rescaled by the
//      softmax correction before each tile.
// With one split the epilogue folds the sink in and writes bf16 output and
// lse; with several it writes the split's normalised fp32 partial and lse.
#include <hip/hip_runtime.h>
#include <math.h>

#include "internal.hpp"

namespace dsv4 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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
__device__ __forceinline__ void dequant8(uint2 raw, float scale, __bf16* v) {
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(raw.x, false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(raw.x, true);
    const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(raw.y, false);
    const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(raw.y, true);
    v[0] = (__bf16)(a[0] * scale);
    v[1] = (__bf16)(a[1] * scale);
    v[2] = (__bf16)(b[0] * scale);
    v[3] = (__bf16)(b[1] * scale);
    v[4] = (__bf16)(c[0] * scale);
    v[5] = (__bf16)(c[1] * scale);
    v[6] = (__bf16)(d[0] * scale);
    v[7] = (__bf16)(d[1] * scale);
}

template <int HG>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(const DecodeParams p) {
    constexpr int MT = HG / 16;              // 16-head MFMA row tiles
    constexpr int TPW = (2 * MT + 3) / 4;    // QK output tiles per wave
    static_assert(HG % 16 == 0 && HG <= kMaxHeadsPerGroup, "head group");

    __shared__ __attribute__((aligned(16))) __bf16 Kn[kTile * kKnLd];
    __shared__ __attribute__((aligned(16))) __bf16 Vt[kD * kVtLd];
    __shared__ float Sb[HG * kSLd];
    __shared__ __attribute__((aligned(16))) __bf16 Pb[HG * kPLd];
    __shared__ __attribute__((aligned(16))) float alpha_s[HG];
    __shared__ float fin_scale[HG];
    __shared__ int64_t ent_doff[kTile];
    __shared__ int64_t ent_soff[kTile];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;

    // Work unit.  Workgroups are handed to the 8 XCDs round-robin; the head
    // groups of one (token, split) are kXcds apart so they land on the same
    // XCD and share its L2 for the rows they both read.
    const int64_t L = blockIdx.x;
    const int x = (int)(L % kXcds);
    const int64_t r8 = L / kXcds;
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

    // q rows of this wave's 16-head QK tile stay in registers: A operand,
    // lane (l16, lg) holds dims 32*ks + 8*lg .. +7 of head 16*mtq + l16.
    const int qk_t0 = wave * TPW;
    const bool has_qk = qk_t0 < 2 * MT;
    const int mtq = has_qk ? qk_t0 / 2 : 0;
    bf16x8 qa[16];
    if (has_qk) {
        const bf16x8* qp = reinterpret_cast<const bf16x8*>(
            p.q + ((int64_t)b * p.H + h0 + 16 * mtq + l16) * kD + 8 * lg);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) qa[ks] = qp[4 * ks];
    }

    // Online-softmax state: head sh is owned by lanes 4*sh .. 4*sh+3, each
    // keeping the same (m, l) in base-2 units.
    const bool smx = tid < 4 * HG;
    const int sh = tid >> 2, sp = tid & 3;
    float m_run = -INFINITY, l_run = 0.f;

    f32x4 acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int t0 = lo; t0 < hi; t0 += kTile) {
        // 1. Resolve entries.
        if (tid < kTile) {
            const int pos = t0 + tid;
            int64_t doff = -1, soff = 0;
            if (pos < hi) {
                const int col = pos < vl ? pos : p.topk + (pos - vl);
                const int32_t idx = p.idx[(int64_t)b * p.idx_stride + col];
                if (idx >= 0) {
                    const int64_t blk = idx / p.bs;
                    const int64_t off = idx % p.bs;
                    int64_t page = -1;
                    if (p.bt) {
                        if (blk < p.max_blocks) {
                            const int32_t pg = p.bt[(int64_t)b * p.bt_stride + blk];
                            if (pg >= 0 && pg < p.num_blocks) page = pg;
                        }
                    } else if (blk < p.num_blocks) {
                        page = blk;
                    }
                    if (page >= 0) {
                        doff = page * p.page_stride + off * kRowData;
                        soff = page * p.page_stride + (int64_t)p.bs * kRowData + off * kRowScale;
                    }
                }
            }
            ent_doff[tid] = doff;
            ent_soff[tid] = soff;
        }
        __syncthreads();

        // 2. Gather + dequantise an 8-row x 8-dim patch per lane.
        {
            const int eg = tid & 3, dc = tid >> 2;   // rows 8eg..8eg+7, dims 8dc..8dc+7
            __bf16 v[8][8];
            if (dc < kDNope / 8) {
                uint2 raw[8];
                uint32_t code[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int64_t doff = ent_doff[8 * eg + i];
                    raw[i] = make_uint2(0u, 0u);
                    code[i] = 127u;
                    if (doff >= 0) {
                        raw[i] = *reinterpret_cast<const uint2*>(p.kv + doff + 8 * dc);
                        code[i] = p.kv[ent_soff[8 * eg + i] + (dc >> 3)];
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) dequant8(raw[i], ue8m0_to_float(code[i]), v[i]);
            } else {
                const int rd = dc - kDNope / 8;      // RoPE dims 448 + 8rd .. +7
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int64_t doff = ent_doff[8 * eg + i];
                    uint2 r0 = make_uint2(0u, 0u), r1 = make_uint2(0u, 0u);
                    if (doff >= 0) {
                        const uint8_t* src = p.kv + doff + kDNope + 16 * rd;
                        r0 = *reinterpret_cast<const uint2*>(src);
                        r1 = *reinterpret_cast<const uint2*>(src + 8);
                    }
                    const uint32_t w[4] = {r0.x, r0.y, r1.x, r1.y};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        v[i][2 * j] = __builtin_bit_cast(__bf16, (uint16_t)(w[j] & 0xFFFFu));
                        v[i][2 * j + 1] = __builtin_bit_cast(__bf16, (uint16_t)(w[j] >> 16));
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                bf16x8 row;
#pragma unroll
                for (int j = 0; j < 8; ++j) row[j] = v[i][j];
                *reinterpret_cast<bf16x8*>(&Kn[(8 * eg + i) * kKnLd + 8 * dc]) = row;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                bf16x8 col;
#pragma unroll
                for (int i = 0; i < 8; ++i) col[i] = v[i][j];
                *reinterpret_cast<bf16x8*>(&Vt[(8 * dc + j) * kVtLd + 8 * eg]) = col;
            }
        }
        __syncthreads();

        // 3. QK: S[head][row] = q . k in base-2 units, -inf where masked.
        if (has_qk) {
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int tau = qk_t0 + j;
                if (tau < 2 * MT) {
                    const int nt = tau & 1;
                    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
                    const __bf16* kp = &Kn[(16 * nt + l16) * kKnLd + 8 * lg];
#pragma unroll
                    for (int ks = 0; ks < 16; ++ks) {
                        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(kp + 32 * ks);
                        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], kb, sacc, 0, 0, 0);
                    }
                    const int n = 16 * nt + l16;
                    const bool ok = ent_doff[n] >= 0;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Sb[(16 * mtq + 4 * lg + r) * kSLd + n] =
                            ok ? sacc[r] * p.qk_scale_log2 : -INFINITY;
                }
            }
        }
        __syncthreads();

        // 4. Online softmax.
        if (smx) {
            float sv[8];
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                sv[i] = Sb[sh * kSLd + 8 * sp + i];
                mx = fmaxf(mx, sv[i]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 1));
            mx = fmaxf(mx, __shfl_xor(mx, 2));
            const float m_new = fmaxf(m_run, mx);
            float alpha = 1.f, psum = 0.f;
            bf16x8 pv;
            if (m_new == -INFINITY) {
#pragma unroll
                for (int i = 0; i < 8; ++i) pv[i] = (__bf16)0.f;
            } else {
                alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 when m_run = -inf
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float e = sv[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[i] - m_new);
                    pv[i] = (__bf16)e;
                    psum += e;
                }
            }
            psum += __shfl_xor(psum, 1);
            psum += __shfl_xor(psum, 2);
            l_run = l_run * alpha + psum;
            m_run = m_new;
            *reinterpret_cast<bf16x8*>(&Pb[sh * kPLd + 8 * sp]) = pv;
            if (sp == 0) alpha_s[sh] = alpha;
        }
        __syncthreads();

        // 5. PV into the wave's 128-dim slab.
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4 al = *reinterpret_cast<const f32x4*>(&alpha_s[16 * mt + 4 * lg]);
            const bf16x8 pa = *reinterpret_cast<const bf16x8*>(&Pb[(16 * mt + l16) * kPLd + 8 * lg]);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const bf16x8 vb = *reinterpret_cast<const bf16x8*>(
                    &Vt[(128 * wave + 16 * nt + l16) * kVtLd + 8 * lg]);
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, acc[mt][nt] * al,
                                                                      0, 0, 0);
            }
        }
        __syncthreads();
    }

    // Epilogue: per-head output scale and lse.
    const bool direct = p.S == 1;
    if (smx && sp == 0) {
        const int h = h0 + sh;
        float scale, lse;
        if (direct && p.sink) {
            const float sk = p.sink[h] * kLog2e;
            const float M = fmaxf(m_run, sk);
            const float em = __builtin_amdgcn_exp2f(m_run - M);
            const float D = l_run * em + __builtin_amdgcn_exp2f(sk - M);
            scale = em / D;
            lse = (M + __builtin_amdgcn_logf(D)) * kLn2;
        } else if (l_run > 0.f) {
            scale = 1.f / l_run;
            lse = (m_run + __builtin_amdgcn_logf(l_run)) * kLn2;
        } else {
            scale = 0.f;
            lse = -INFINITY;
        }
        fin_scale[sh] = scale;
        if (direct) {
            if (p.lse) p.lse[(int64_t)b * p.H + h] = lse;
        } else {
            p.part_lse[((int64_t)b * p.H + h) * p.S + s] = lse;
        }
    }
    __syncthreads();

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int hl = 16 * mt + 4 * lg + r;
            const float sc = fin_scale[hl];
            const int64_t row = (int64_t)b * p.H + h0 + hl;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const int d = 128 * wave + 16 * nt + l16;
                const float val = acc[mt][nt][r] * sc;
                if (direct)
                    p.out[row * kD + d] = __builtin_bit_cast(uint16_t, (__bf16)val);
                else
                    p.part_o[(row * p.S + s) * kD + d] = val;
            }
        }
    }
}

// Merge of split partials with the sink; one workgroup per (token, head),
// 4 output dims per lane.
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const CombineParams p) {
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % p.H);
    const float* ls = p.part_lse + bh * p.S;
    const float sink = p.sink ? p.sink[h] : -INFINITY;
    float M = sink;
    for (int s = 0; s < p.S; ++s) M = fmaxf(M, ls[s]);
    const int d = threadIdx.x * 4;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float lse = -INFINITY;
    if (M != -INFINITY) {
        float D = 0.f;
        for (int s = 0; s < p.S; ++s) {
            const float l = ls[s];
            if (l == -INFINITY) continue;
            const float w = __builtin_amdgcn_exp2f((l - M) * kLog2e);
            D += w;
            o += w * *reinterpret_cast<const f32x4*>(p.part_o + (bh * p.S + s) * kD + d);
        }
        if (p.sink) D += __builtin_amdgcn_exp2f((sink - M) * kLog2e);
        o *= 1.f / D;
        lse = M + __builtin_amdgcn_logf(D) * kLn2;
    }
    uint2 packed;
    packed.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[0]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[1]) << 16);
    packed.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[2]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o[3]) << 16);
    *reinterpret_cast<uint2*>(p.out + bh * kD + d) = packed;
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
    const int64_t grid = (int64_t)p.B * p.H;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)grid), dim3(kCombineThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace dsv4
