/*
 * Plain fp64 CPU oracle for sparse FP8 MLA decode over an fp8_ds_mla cache.
 *
 * TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
 * baseline leg may call it; the product path never does.  No code, header,
 * table or constant is shared with the HIP library.
 *
 * Sources (titles of the pages the method is described on):
 *   [vLLM-52212]  vLLM PR #52212, gfx950 DSV4 sparse decode kernel page
 *   [SGL-26208]   SGLang PR #26208 report, "[AMD] Dsv4/pr2 compressor opt"
 *   [vLLM-41217]  vLLM PR #41217 report, "[ROCm][Deepseek] dsv3.2 further
 *                 optimization"
 *   [SGL-26383]   SGLang PR #26383 page (DSV4 MTP graph capture on ROCm)
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes of the repository):
 *   - FP8 is OCP E4M3FN (bias 7, no infinities, S.1111.111 = NaN);
 *   - a UE8M0 code c means 2^(c-127), code 255 is NaN;
 *   - code g scales NoPE dims [64g, 64g+64), the eighth scale byte is padding;
 *   - V is the same 512 dequantised dims as K;
 *   - the sink is a per-head logit in natural units that joins the softmax
 *     denominator with no value row; lse = ln(sum_valid e^s + e^sink);
 *   - valid_len masks main positions [valid_len, topk) only, clamped to
 *     [0, topk]; SWA positions are never masked by it;
 *   - an index is invalid when negative or when its page does not resolve.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define ORC_D 512
#define ORC_DNOPE 448
#define ORC_DROPE 64
#define ORC_ROW_DATA 576
#define ORC_ROW_SCALE 8

/* OCP 8-bit E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits; the
 * all-ones exponent with all-ones mantissa is NaN and there is no infinity.
 * [SGL-26208] key source snippets (the FP8 NoPE bytes of a DSV4 row). */
double orc_e4m3fn(uint8_t code) {
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                  /* m/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* UE8M0 scale: an unsigned power-of-two exponent, 2^(code-127); 255 = NaN.
 * [vLLM-52212] implementation item 3 and the writer snippet (codes are
 * clamped to at most 254 when the writer sanitises). */
double orc_ue8m0(uint8_t code) {
    if (code == 255) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* bfloat16: sign, 8 exponent bits (bias 127), 7 mantissa bits. */
double orc_bf16(uint16_t bits) {
    int sign = bits >> 15;
    int e = (bits >> 7) & 0xFF;
    int m = bits & 0x7F;
    double v;
    if (e == 0xFF) {
        if (m) return NAN;
        v = INFINITY;
    } else if (e == 0) {
        v = ldexp((double)m, -133);                /* m/128 * 2^-126 */
    } else {
        v = ldexp(1.0 + (double)m / 128.0, e - 127);
    }
    return sign ? -v : v;
}

/* Page lookup: block = idx / block_size, offset = idx % block_size, page from
 * the block table; a negative index, a block past the table or a page outside
 * the pool names no row.  [SGL-26208] gather+dequant kernel (-1 invalid,
 * block index and in-block offset), [vLLM-41217] conversion kernel (block
 * range check), [vLLM-52212] cp-gather snippet (pages outside [0, NUM_BLOCKS)
 * are invalid). */
int orc_resolve(const orc_desc* d, const int32_t* block_table, int32_t b, int32_t idx,
                int64_t* page, int32_t* off) {
    int64_t blk, p;
    if (idx < 0) return 0;
    blk = (int64_t)idx / d->block_size;
    if (block_table) {
        if (blk >= d->max_blocks_per_seq) return 0;
        p = block_table[(int64_t)b * d->block_table_stride + blk];
        if (p < 0 || p >= d->num_blocks) return 0;
    } else {
        p = blk;
        if (p >= d->num_blocks) return 0;
    }
    *page = p;
    *off = (int32_t)((int64_t)idx % d->block_size);
    return 1;
}

/* Row bytes at page*stride + off*576; its 8 scale bytes at
 * page*stride + block_size*576 + off*8.  NoPE dim j = E4M3FN(byte j) times
 * UE8M0(code j/64); RoPE dim r = bf16 from bytes 448+2r (low) and 449+2r.
 * [SGL-26208] DSV4 constants and the gather+dequant address arithmetic.
 * With d->scrub, a dimension whose value is not finite (an FP8 NaN byte, a
 * NaN scale code, a NaN or infinite RoPE value) is read as 0: the legacy
 * element-wise clearing the decode keeps when the cache is not trusted to
 * be NaN-free ([vLLM-52212] implementation item 3 and the provenance gate
 * in its ROCm entry-layer snippet). */
void orc_dequant_row(const orc_desc* d, const uint8_t* kv, int64_t page, int32_t off,
                     double* out) {
    const uint8_t* data = kv + page * d->page_stride + (int64_t)off * ORC_ROW_DATA;
    const uint8_t* scales = kv + page * d->page_stride + (int64_t)d->block_size * ORC_ROW_DATA +
                            (int64_t)off * ORC_ROW_SCALE;
    int j, r;
    for (j = 0; j < ORC_DNOPE; ++j) out[j] = orc_e4m3fn(data[j]) * orc_ue8m0(scales[j / 64]);
    for (r = 0; r < ORC_DROPE; ++r) {
        uint16_t bits = (uint16_t)(data[ORC_DNOPE + 2 * r] | (data[ORC_DNOPE + 2 * r + 1] << 8));
        out[ORC_DNOPE + r] = orc_bf16(bits);
    }
    if (d->scrub)
        for (j = 0; j < ORC_D; ++j)
            if (!isfinite(out[j])) out[j] = 0.0;
}

/* valid_len clamps to [0, topk]; NULL means the whole main list. */
static int32_t eff_main_len(const orc_desc* d, const int32_t* valid_len, int32_t b) {
    int32_t vl;
    if (!valid_len) return d->topk;
    vl = valid_len[b];
    if (vl < 0) vl = 0;
    if (vl > d->topk) vl = d->topk;
    return vl;
}

/* Column of the index row at position p of the effective list
 * main[0:vl] ++ swa. */
static int32_t eff_to_col(const orc_desc* d, int32_t vl, int32_t p) {
    return p < vl ? p : d->topk + (p - vl);
}

typedef struct {
    const orc_desc* d;
    const uint16_t* q;
    const uint8_t* kv;
    const int32_t* bt;
    const orc_desc* d_swa;            /* second pool of the SWA entries, or NULL */
    const uint8_t* kv_swa;
    const int32_t* bt_swa;
    const int32_t* idx;
    const int32_t* valid_len;
    const float* sink;
    int32_t num_splits;
    double* out;
    double* lse;
    int64_t item_begin, item_end;     /* flattened (b, h) range */
    int64_t n_valid;                  /* valid entries of the rows this worker started */
} orc_job;

/* One (b, h): sparse softmax attention with sink over the valid entries.
 * rows[p] holds the dequantised row at effective position p, valid[p] says
 * whether it counts.  [vLLM-52212] implementation item 1 (one 512-wide QK
 * dot over NoPE+RoPE, masked tail, sink and invalid-index semantics kept),
 * [SGL-26208] unified kernel interface (Output and LSE with an attention
 * sink), review highlights (a masked or -inf score adds exactly nothing). */
static void attend_one(const orc_job* J, int32_t b, int32_t h, int32_t eff_len,
                       const double* rows, const unsigned char* valid, double* qd,
                       double* s, double* acc) {
    const orc_desc* d = J->d;
    double* o = J->out + ((int64_t)b * d->H + h) * ORC_D;
    double* lse = J->lse + (int64_t)b * d->H + h;
    const int has_sink = J->sink != NULL;
    const double sink = has_sink ? (double)J->sink[h] : -INFINITY;
    int32_t p, j, S, sidx;

    for (j = 0; j < ORC_D; ++j) qd[j] = orc_bf16(J->q[((int64_t)b * d->H + h) * ORC_D + j]);
    for (p = 0; p < eff_len; ++p) {
        double dot = 0.0;
        if (!valid[p]) continue;
        for (j = 0; j < ORC_D; ++j) dot += qd[j] * rows[(int64_t)p * ORC_D + j];
        s[p] = d->sm_scale * dot;
    }

    S = J->num_splits;
    if (S <= 0) {
        /* The definition: M = max(s, sink); D = sum e^(s-M) + e^(sink-M). */
        double M = -INFINITY, D = 0.0;
        int any = 0;
        for (p = 0; p < eff_len; ++p)
            if (valid[p] && (!any || s[p] > M)) {
                M = s[p];
                any = 1;
            }
        if (!any) {
            for (j = 0; j < ORC_D; ++j) o[j] = 0.0;
            *lse = sink;
            return;
        }
        if (has_sink && sink > M) M = sink;
        for (j = 0; j < ORC_D; ++j) acc[j] = 0.0;
        for (p = 0; p < eff_len; ++p) {
            double w;
            if (!valid[p]) continue;
            w = exp(s[p] - M);
            D += w;
            for (j = 0; j < ORC_D; ++j) acc[j] += w * rows[(int64_t)p * ORC_D + j];
        }
        if (has_sink) D += exp(sink - M);
        for (j = 0; j < ORC_D; ++j) o[j] = acc[j] / D;
        *lse = M + log(D);
        return;
    }

    /* Split form: contiguous chunks of the effective list, each reduced to a
     * normalised partial and its log-sum-exp, then merged with the sink.
     * [vLLM-52212] implementation item 2 (split-K with per-row splits),
     * [SGL-26208] implementation item 3 (split-K over the top-k axis). */
    {
        int32_t chunk = (eff_len + S - 1) / S;
        double* po = acc;                 /* S partials of 512 */
        double* plse = acc + (int64_t)S * ORC_D;
        double M, D;
        for (sidx = 0; sidx < S; ++sidx) {
            int32_t lo = sidx * chunk, hi = lo + chunk, any = 0;
            double m = 0.0, l = 0.0;
            double* ps = po + (int64_t)sidx * ORC_D;
            if (chunk == 0) lo = hi = 0;
            if (hi > eff_len) hi = eff_len;
            for (j = 0; j < ORC_D; ++j) ps[j] = 0.0;
            for (p = lo; p < hi; ++p)
                if (valid[p] && (!any || s[p] > m)) { m = s[p]; any = 1; }
            if (!any) { plse[sidx] = -INFINITY; continue; }
            for (p = lo; p < hi; ++p) {
                double w;
                if (!valid[p]) continue;
                w = exp(s[p] - m);
                l += w;
                for (j = 0; j < ORC_D; ++j) ps[j] += w * rows[(int64_t)p * ORC_D + j];
            }
            for (j = 0; j < ORC_D; ++j) ps[j] /= l;
            plse[sidx] = m + log(l);
        }
        M = sink;
        for (sidx = 0; sidx < S; ++sidx)
            if (plse[sidx] > M) M = plse[sidx];
        if (M == -INFINITY) {
            for (j = 0; j < ORC_D; ++j) o[j] = 0.0;
            *lse = sink;
            return;
        }
        D = has_sink ? exp(sink - M) : 0.0;
        for (j = 0; j < ORC_D; ++j) o[j] = 0.0;
        for (sidx = 0; sidx < S; ++sidx) {
            double w;
            if (plse[sidx] == -INFINITY) continue;
            w = exp(plse[sidx] - M);
            D += w;
            for (j = 0; j < ORC_D; ++j) o[j] += w * po[(int64_t)sidx * ORC_D + j];
        }
        for (j = 0; j < ORC_D; ++j) o[j] /= D;
        *lse = M + log(D);
    }
}

static void* orc_worker(void* arg) {
    orc_job* J = (orc_job*)arg;
    const orc_desc* d = J->d;
    const int32_t Kt = d->topk + d->swa;
    const int32_t S = J->num_splits > 0 ? J->num_splits : 0;
    double* rows = (double*)malloc(sizeof(double) * (size_t)(Kt > 0 ? Kt : 1) * ORC_D);
    unsigned char* valid = (unsigned char*)malloc((size_t)(Kt > 0 ? Kt : 1));
    double* qd = (double*)malloc(sizeof(double) * ORC_D);
    double* s = (double*)malloc(sizeof(double) * (size_t)(Kt > 0 ? Kt : 1));
    double* acc = (double*)malloc(sizeof(double) * ((size_t)(S + 1) * ORC_D + (size_t)S + 1));
    int32_t cur_b = -1, eff_len = 0;
    int64_t it;
    J->n_valid = 0;
    for (it = J->item_begin; it < J->item_end; ++it) {
        int32_t b = (int32_t)(it / d->H), h = (int32_t)(it % d->H);
        if (b != cur_b) {
            /* The s_q query tokens of a sequence share its block-table row
             * and top-k length ([SGL-26208] gather+dequant kernel: the
             * length of token t is read at t // s_q). */
            const int32_t seq = d->s_q > 1 ? b / d->s_q : b;
            int32_t vl = eff_main_len(d, J->valid_len, seq), p;
            cur_b = b;
            eff_len = vl + d->swa;
            for (p = 0; p < eff_len; ++p) {
                int32_t col = eff_to_col(d, vl, p);
                int32_t idx = J->idx[(int64_t)b * Kt + col];
                /* With a second pool, SWA entries (columns >= topk) name its
                 * rows through its own block table and geometry. */
                const int use_swa = J->d_swa != NULL && col >= d->topk;
                const orc_desc* dp = use_swa ? J->d_swa : d;
                const uint8_t* kvp = use_swa ? J->kv_swa : J->kv;
                const int32_t* btp = use_swa ? J->bt_swa : J->bt;
                int64_t page;
                int32_t off;
                valid[p] = (unsigned char)orc_resolve(dp, btp, seq, idx, &page, &off);
                if (valid[p]) orc_dequant_row(dp, kvp, page, off, rows + (int64_t)p * ORC_D);
            }
            if (h == 0)
                for (p = 0; p < eff_len; ++p) J->n_valid += valid[p];
        }
        attend_one(J, b, h, eff_len, rows, valid, qd, s, acc);
    }
    free(rows); free(valid); free(qd); free(s); free(acc);
    return NULL;
}

int64_t orc_sparse_decode(const orc_desc* d, const uint16_t* q, const uint8_t* kv,
                          const int32_t* block_table, const int32_t* topk_idx,
                          const int32_t* valid_len, const float* sink, int32_t num_splits,
                          double* out, double* lse, int32_t nthreads) {
    return orc_sparse_decode_dual(d, NULL, q, kv, block_table, NULL, NULL, topk_idx, valid_len,
                                  sink, num_splits, out, lse, nthreads);
}

/* Dual-pool decode: the SWA entries resolve in a second fp8_ds_mla pool
 * with its own block table, block size and page stride (DeepSeek-V4 keeps
 * the sliding-window cache apart from the compressed "extra" cache the main
 * top-k entries index: [vLLM-52212] implementation item 1, main/SWA work,
 * and item 3, the extra cache).  d_swa NULL: one pool. */
int64_t orc_sparse_decode_dual(const orc_desc* d, const orc_desc* d_swa, const uint16_t* q,
                               const uint8_t* kv, const int32_t* block_table,
                               const uint8_t* kv_swa, const int32_t* bt_swa,
                               const int32_t* topk_idx, const int32_t* valid_len,
                               const float* sink, int32_t num_splits, double* out, double* lse,
                               int32_t nthreads) {
    int64_t items = (int64_t)d->B * d->H, total = 0;
    int32_t t, nt = nthreads < 1 ? 1 : nthreads;
    orc_job* jobs;
    pthread_t* th;
    if (items <= 0) return 0;
    if (nt > items) nt = (int32_t)items;
    jobs = (orc_job*)calloc((size_t)nt, sizeof(orc_job));
    th = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
    for (t = 0; t < nt; ++t) {
        orc_job* J = &jobs[t];
        J->d = d; J->q = q; J->kv = kv; J->bt = block_table; J->idx = topk_idx;
        J->d_swa = d_swa; J->kv_swa = kv_swa; J->bt_swa = bt_swa;
        J->valid_len = valid_len; J->sink = sink; J->num_splits = num_splits;
        J->out = out; J->lse = lse;
        J->item_begin = items * t / nt;
        J->item_end = items * (t + 1) / nt;
    }
    for (t = 1; t < nt; ++t) pthread_create(&th[t], NULL, orc_worker, &jobs[t]);
    orc_worker(&jobs[0]);
    for (t = 1; t < nt; ++t) pthread_join(th[t], NULL);
    /* Each b's valid entries are counted by the worker that met its h == 0. */
    for (t = 0; t < nt; ++t) total += jobs[t].n_valid;
    free(jobs); free(th);
    return total;
}

/* out = fill when the index is negative, its block is outside
 * [0, max_blocks_per_req), the request is outside the table, the page entry
 * is negative or the slot does not fit in int32; else page*block_size + off,
 * computed in 64 bits.  Dense rows, or ragged rows stored from cu[t].
 * [vLLM-41217] key source snippets, the req-index to global-index kernel
 * (the fill there is 0; here it is an argument, and a negative page entry
 * also yields the fill). */
void orc_convert_req_index_to_global(const int32_t* req_id, int32_t num_reqs,
                                     const int32_t* block_table, int64_t bt_stride,
                                     int32_t max_blocks_per_req, const int32_t* token_indices,
                                     int64_t ti_stride, int32_t num_tokens, int32_t width,
                                     int32_t block_size, const int32_t* cu_seqlens,
                                     int32_t invalid_fill, int32_t* out) {
    int32_t t, i;
    for (t = 0; t < num_tokens; ++t) {
        int32_t req = req_id ? req_id[t] : t;
        int64_t base, n;
        if (cu_seqlens) {
            base = cu_seqlens[t];
            n = (int64_t)cu_seqlens[t + 1] - cu_seqlens[t];
            if (n > width) n = width;
        } else {
            base = (int64_t)t * width;
            n = width;
        }
        for (i = 0; i < n; ++i) {
            int32_t idx = token_indices[(int64_t)t * ti_stride + i];
            int64_t v = invalid_fill;
            if (idx >= 0 && req >= 0 && req < num_reqs) {
                int64_t blk = (int64_t)idx / block_size;
                int64_t off = (int64_t)idx % block_size;
                if (blk < max_blocks_per_req) {
                    int64_t page = block_table[(int64_t)req * bt_stride + blk];
                    if (page >= 0) {
                        int64_t g = page * block_size + off;
                        if (g <= 2147483647LL) v = g;
                    }
                }
            }
            if (cu_seqlens && (base + i < 0 || base + i >= cu_seqlens[num_tokens])) continue;
            out[base + i] = (int32_t)v;
        }
    }
}

/* ------------------------------------------------------------ cache writer */

/* Nearest E4M3FN code to a finite v with |v| <= 448: the non-negative codes
 * 0x00..0x7E are the whole finite grid; the closest one wins and a tie goes
 * to the even code (mantissa LSB 0).  The sign bit is v's, so -0 and
 * negative values that round to zero give 0x80. */
static uint8_t orc_encode_e4m3fn(double v) {
    double a = fabs(v), best_d = INFINITY;
    int c, best = 0;
    for (c = 0; c <= 0x7E; ++c) {
        double d = fabs(orc_e4m3fn((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best_d = d;
            best = c;
        }
    }
    return (uint8_t)(best | (signbit(v) ? 0x80 : 0));
}

/* Quantise one 512-wide bf16 row into the fp8_ds_mla row format.
 *
 * NoPE group g (dims [64g, 64g+64)): a = the largest |x| of the group, NaN
 * elements left out; its UE8M0 code is the smallest c in [0, cap] with
 * a <= 448 * 2^(c-127) (cap when none is), the value divided by the scale
 * then lands in the FP8 range; each element is stored as the E4M3FN
 * rounding of x * 2^(127-c) clamped to [-448, 448], a NaN element as 0x7F.
 * cap = 254 with sanitize, else 255 (a NaN scale).  RoPE dims are stored as
 * the input bf16; with sanitize a NaN or infinite RoPE value is stored as
 * +0.  Scale byte 7 is 0.
 * [vLLM-52212] the sanitising writer snippet (code clamped to [0, 254]
 * instead of [0, 255]; non-finite RoPE values normalised to 0, so the
 * decoder can skip its scrub); the smallest-sufficient-code rule is the
 * reading taken where the pages do not print the amax -> code step. */
void orc_quantize_row(const uint16_t* x, int32_t sanitize, uint8_t* data, uint8_t* scales) {
    const int cap = sanitize ? 254 : 255;
    int g, j, c, r;
    for (g = 0; g < ORC_DNOPE / 64; ++g) {
        double a = 0.0;
        for (j = 64 * g; j < 64 * g + 64; ++j) {
            double v = orc_bf16(x[j]);
            if (!isnan(v) && fabs(v) > a) a = fabs(v);
        }
        for (c = 0; c < cap; ++c)
            if (a <= 448.0 * ldexp(1.0, c - 127)) break;
        scales[g] = (uint8_t)c;
        for (j = 64 * g; j < 64 * g + 64; ++j) {
            double v = orc_bf16(x[j]);
            if (isnan(v)) {
                data[j] = 0x7F;
                continue;
            }
            v = ldexp(v, 127 - c);
            if (v > 448.0) v = 448.0;
            if (v < -448.0) v = -448.0;
            data[j] = orc_encode_e4m3fn(v);
        }
    }
    scales[7] = 0;
    for (r = 0; r < ORC_DROPE; ++r) {
        uint16_t bits = x[ORC_DNOPE + r];
        if (sanitize && !isfinite(orc_bf16(bits))) bits = 0;
        data[ORC_DNOPE + 2 * r] = (uint8_t)(bits & 0xFF);
        data[ORC_DNOPE + 2 * r + 1] = (uint8_t)(bits >> 8);
    }
}

/* Store n rows at global slots: slot s is row s % block_size of page
 * s / block_size (the same addressing the decode reads); a negative slot or
 * one past the pool is skipped. */
void orc_store_rows(const uint16_t* rows, int64_t row_stride, const int64_t* slots, int64_t n,
                    uint8_t* kv, int32_t block_size, int64_t num_blocks, int64_t page_stride,
                    int32_t sanitize) {
    int64_t i;
    for (i = 0; i < n; ++i) {
        int64_t s = slots[i], page, off;
        if (s < 0) continue;
        page = s / block_size;
        off = s % block_size;
        if (page >= num_blocks) continue;
        orc_quantize_row(rows + i * row_stride, sanitize,
                         kv + page * page_stride + off * ORC_ROW_DATA,
                         kv + page * page_stride + (int64_t)block_size * ORC_ROW_DATA +
                             off * ORC_ROW_SCALE);
    }
}
