/*
 * Plain fp64 CPU oracle for sparse FP8 MLA decode over an fp8_ds_mla cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this code; the product
 * path (the HIP library and its Python binding) never does.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * What it computes is the plain definition the fast path must reach: sparse
 * softmax attention with an attention-sink logit over the gathered,
 * dequantised cache rows, and the block-table index conversion.  Every
 * function names the page passage it follows in oracle.c.
 */
#ifndef DSV4_ORACLE_H
#define DSV4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t B;                   /* query tokens, one per sequence           */
    int32_t H;                   /* heads                                    */
    int32_t topk;                /* main entries per token                   */
    int32_t swa;                 /* sliding-window entries per token         */
    int32_t block_size;          /* slots per page                           */
    int32_t max_blocks_per_seq;  /* usable block-table columns               */
    int64_t num_blocks;          /* pages in the pool                        */
    int64_t block_table_stride;  /* elements between block-table rows        */
    int64_t page_stride;         /* bytes between pages                      */
    double sm_scale;             /* softmax scale on q.k (not on the sink)   */
    int32_t scrub;               /* 1: every dequantised element that is not
                                    finite is read as 0 (decode-time scrub)  */
    int32_t s_q;                 /* query tokens per sequence (<= 1: one);
                                    token b reads block-table row and
                                    valid_len entry b / s_q                  */
} orc_desc;

/* Scalar decoders. */
double orc_e4m3fn(uint8_t code);
double orc_ue8m0(uint8_t code);
double orc_bf16(uint16_t bits);

/* Entry resolution: 1 and (page, off) when slot idx of row b names a cache
 * row, 0 otherwise.  block_table may be NULL (idx is then a pool slot). */
int orc_resolve(const orc_desc* d, const int32_t* block_table, int32_t b, int32_t idx,
                int64_t* page, int32_t* off);

/* Dequantise one row (448 NoPE + 64 RoPE) into out[512]. */
void orc_dequant_row(const orc_desc* d, const uint8_t* kv, int64_t page, int32_t off,
                     double* out);

/* Whole decode.  q: bf16 bits [B,H,512]; topk_idx [B, topk+swa]; valid_len
 * [B] or NULL; sink [H] or NULL.  out [B,H,512] and lse [B,H] in fp64.
 * num_splits = 0 computes the plain definition; num_splits > 0 computes
 * per-chunk partials over the effective list and merges them by
 * log-sum-exp.  nthreads >= 1.  Returns the number of valid entries. */
int64_t orc_sparse_decode(const orc_desc* d, const uint16_t* q, const uint8_t* kv,
                          const int32_t* block_table, const int32_t* topk_idx,
                          const int32_t* valid_len, const float* sink, int32_t num_splits,
                          double* out, double* lse, int32_t nthreads);

/* Dual-pool decode: entries at columns >= topk (the SWA part) resolve and
 * dequantise in the second pool (d_swa geometry, kv_swa, bt_swa); d_swa
 * NULL means one pool.  Other arguments as orc_sparse_decode. */
int64_t orc_sparse_decode_dual(const orc_desc* d, const orc_desc* d_swa, const uint16_t* q,
                               const uint8_t* kv, const int32_t* block_table,
                               const uint8_t* kv_swa, const int32_t* bt_swa,
                               const int32_t* topk_idx, const int32_t* valid_len,
                               const float* sink, int32_t num_splits, double* out, double* lse,
                               int32_t nthreads);

/* Req-local -> global slot conversion.  Dense when cu_seqlens is NULL
 * (out[t*width + i]); ragged otherwise (out[cu[t] + i], i < cu[t+1]-cu[t]).
 * req_id may be NULL (request t for token t). */
void orc_convert_req_index_to_global(const int32_t* req_id, int32_t num_reqs,
                                     const int32_t* block_table, int64_t bt_stride,
                                     int32_t max_blocks_per_req, const int32_t* token_indices,
                                     int64_t ti_stride, int32_t num_tokens, int32_t width,
                                     int32_t block_size, const int32_t* cu_seqlens,
                                     int32_t invalid_fill, int32_t* out);

/* Cache writer: quantise one bf16 row (448 NoPE + 64 RoPE) into 576 data
 * bytes and 8 scale bytes; sanitize = 1 caps codes at 254 and stores
 * non-finite RoPE values as 0. */
void orc_quantize_row(const uint16_t* x, int32_t sanitize, uint8_t* data, uint8_t* scales);

/* Quantise-and-store n rows (bf16, row_stride elements apart) at global
 * slots; negative slots and slots past the pool are skipped. */
void orc_store_rows(const uint16_t* rows, int64_t row_stride, const int64_t* slots, int64_t n,
                    uint8_t* kv, int32_t block_size, int64_t num_blocks, int64_t page_stride,
                    int32_t sanitize);

#ifdef __cplusplus
}
#endif
#endif
