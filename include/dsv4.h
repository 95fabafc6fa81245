/*
 * dsv4.h -- C ABI of the MI355X (gfx950) sparse FP8 MLA decode library.
 *
 * The library computes DeepSeek-V4-style sparse MLA decode over an FP8
 * "fp8_ds_mla" latent KV cache, and the req-local -> global block-table
 * index conversion that feeds it.  Sources (page titles):
 *   vLLM PR #52212, gfx950 DSV4 sparse decode kernel page;
 *   SGLang PR #26208 report, "[AMD] Dsv4/pr2 compressor opt";
 *   vLLM PR #41217 report, "[ROCm][Deepseek] dsv3.2 further optimization";
 *   SGLang PR #26383 page (fused no-split-K attention at >= 256 tokens).
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The
 *     library allocates nothing, keeps no pointer after a call returns,
 *     never synchronises and never throws across this ABI.
 *   - Work is enqueued asynchronously on `stream` (NULL = the null stream).
 *   - The return value is a dsv4_status.  On failure nothing was launched
 *     (except DSV4_ERR_HIP, where a launch failed) and dsv4_last_error()
 *     describes the problem for the calling thread.
 *   - Bad data (negative indices, blocks past the table, page entries
 *     outside the pool, valid_len outside [0, topk]) is masked, never an
 *     error: such entries simply do not take part.  Bad shapes, strides,
 *     alignments or NULL required pointers are errors.
 *   - Given the same arguments (including the split count) results are
 *     bitwise reproducible: no atomics take part in any sum.
 */
#ifndef DSV4_H
#define DSV4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */

typedef enum dsv4_status {
    DSV4_OK = 0,
    DSV4_ERR_INVALID_ARGUMENT = 1,   /* NULL required pointer, bad shape/stride/alignment */
    DSV4_ERR_NOT_SUPPORTED = 2,      /* a shape the kernels have no variant for (no valid
                                        descriptor returns it at present)               */
    DSV4_ERR_WORKSPACE_TOO_SMALL = 3,
    DSV4_ERR_HIP = 4                 /* a kernel launch failed; see dsv4_last_error()     */
} dsv4_status;

/* Human-readable name of a status value (static storage). */
const char* dsv4_status_string(int status);

/* Message of the last failed call made by this thread ("" if none). */
const char* dsv4_last_error(void);

/* ------------------------------------------------------- cache geometry */

/* One cache row: 448 FP8-E4M3FN NoPE bytes then 64 little-endian bf16 RoPE
 * values (576 bytes), plus 8 scale bytes: UE8M0 code g scales NoPE dims
 * [64g, 64g+64) by 2^(code-127); the eighth byte is padding.  A page of
 * block_size rows stores the data rows first and the scale words after
 * them: row `off` of page `page` is at page*page_stride + off*576, its
 * scales at page*page_stride + block_size*576 + off*8.
 * (SGLang PR #26208 report, key source snippets: the DSV4 constants and the
 * gather+dequant address arithmetic.) */
#define DSV4_D_QK 512
#define DSV4_D_NOPE 448
#define DSV4_D_ROPE 64
#define DSV4_ROW_DATA_BYTES 576
#define DSV4_ROW_SCALE_BYTES 8
#define DSV4_MAX_SPLITS 64

/* ------------------------------------------------------------ decode */

/* Decode flags (dsv4_decode_desc.flags).
 *
 * DSV4_DECODE_SCRUB: every dequantised K/V element that is not finite (an
 * FP8 NaN byte, scale code 255, a product beyond the bf16 range, a NaN or
 * infinite RoPE value) is read as 0 before it enters any product.  For a
 * cache whose writer is not known to keep it NaN-free; a cache whose writer
 * sanitises non-finite values runs without it, at no cost.  (vLLM PR #52212 page, implementation item 3: element-wise
 * clearing of NoPE/RoPE is the legacy behaviour, dropped when the cache's
 * provenance guarantees finite values; its ROCm entry-layer snippet gates
 * the choice on a flag.)  Other bits are reserved and must be 0. */
#define DSV4_DECODE_SCRUB 0x1u

/* DSV4_DECODE_PIPELINED: run the pipelined partial kernel even where the plan
 * would pick the short-split kernel (splits of at most 128 entries); results
 * differ only by rounding.  For comparing the two kernels. */
#define DSV4_DECODE_PIPELINED 0x2u

/* DSV4_DECODE_BALANCE: spread the splits over the tokens by their lengths,
 * for batches whose valid_len differ from token to token.  The plan keeps
 * its B * S split workgroups per head group (S forced or chosen as usual);
 * the kernel reads valid_len at run time and gives token b
 *   n_b = max(1, ceil(eff_b / (32 T))) splits,  eff_b = valid_len[b] + swa,
 * with T the fewest 32-entry tiles per split for which sum_b n_b <= B * S and
 * every n_b fits the row's split slots; each token's effective list is cut
 * into n_b contiguous chunks of whole tiles as usual.  The partials then hold
 * S' = min(64, S + ceil(S / 4)) split slots per (token, head) row
 * (plan.num_splits = S', plan.balanced_splits = S); slots a token leaves
 * unused hold lse = -inf.  It applies to plans that run the pipelined kernel
 * with S >= 2 and batch <= 64 (plan.balanced_splits != 0 then) and is
 * ignored otherwise; the global slots of dsv4_sparse_decode_with_slots then
 * come from a conversion launch, and dsv4_gather_floor and dsv4_dense_decode
 * reject it.  (vLLM PR #52212 page, implementation item 2: a fixed grid whose
 * rows take their active splits at run time.) */
#define DSV4_DECODE_BALANCE 0x4u

/* Provenance gate: the decode flags a cache of this provenance needs.
 * Returns 0 (the scrub may be skipped) only when every condition holds:
 * the cache is in the fp8_ds_mla format, no KV transfer (another engine,
 * another process) wrote into it, the extra (compressed) cache is present,
 * and its writer sanitised (dsv4_quantize_store with DSV4_STORE_SANITIZE,
 * or an equivalent writer); otherwise DSV4_DECODE_SCRUB.  Host-only; never
 * fails.  (vLLM PR #52212 page, implementation item 3 and the ROCm
 * entry-layer snippet: the NaN-free trust gate, whose gfx950 clause stands
 * for the sanitising writer that platform enables.) */
uint32_t dsv4_decode_flags_for_cache(int32_t cache_is_fp8_ds_mla, int32_t has_kv_transfer,
                                     int32_t has_extra_cache, int32_t writer_sanitizes);

typedef struct dsv4_decode_desc {
    int32_t batch;               /* B: query tokens (rows of q / topk_idx / out), >= 1 */
    int32_t num_heads;           /* H: multiple of 16 in [16, 128]                   */
    int32_t topk;                /* main entries per token, >= 0                     */
    int32_t swa;                 /* sliding-window entries per token, >= 0           */
    int32_t block_size;          /* slots per page, >= 1                             */
    int32_t max_blocks_per_seq;  /* usable block_table columns (ignored if no table) */
    int64_t num_blocks;          /* pages in kv_cache, >= 1                          */
    int64_t block_table_stride;  /* elements between block_table rows                */
    int64_t page_stride;         /* bytes between pages: >= block_size*584, mult. of 8 */
    int64_t topk_idx_stride;     /* elements between topk_idx rows; 0 = topk + swa   */
    float sm_scale;              /* multiplies q.k (never the sink)                  */
    uint32_t flags;              /* DSV4_DECODE_* bits; 0 = none                     */
    int32_t tokens_per_seq;      /* s_q: query tokens per sequence (0 or 1 = one);
                                    batch must be a multiple of it                   */
    void* workspace;             /* device scratch for split partials (may be NULL
                                    when the call needs none)                        */
    size_t workspace_bytes;      /* its size                                         */
} dsv4_decode_desc;

/* What a decode call will launch.  Filled on the host; needs no GPU. */
typedef struct dsv4_plan {
    int32_t num_splits;          /* S used (forced, or chosen by the selector); split
                                    slots per row of the partials (see balanced_splits) */
    int32_t heads_per_group;     /* heads one workgroup serves                       */
    int32_t head_groups;         /* H / heads_per_group                              */
    int32_t tile_entries;        /* cache rows per pipeline tile                     */
    int64_t grid_partial;        /* workgroups of the partial kernel                 */
    int32_t block_partial;       /* threads per partial workgroup                    */
    int64_t grid_combine;        /* workgroups of the combine kernel (0 if S == 1)   */
    int32_t block_combine;       /* threads per combine workgroup                    */
    size_t workspace_bytes;      /* scratch the call needs (0 if S == 1)             */
    size_t lds_bytes;            /* LDS per partial workgroup                        */
    int32_t partial_kernel;      /* DSV4_KERNEL_PIPELINED or DSV4_KERNEL_SHORT       */
    int32_t balanced_splits;     /* DSV4_DECODE_BALANCE in effect: the split budget S
                                    per token (num_splits is then the split slots per
                                    row, S + ceil(S/4)); 0 = uniform splits          */
} dsv4_plan;

/* Partial kernels (dsv4_plan.partial_kernel).  The short-split kernel serves
 * plans whose splits hold at most 128 entries with 16, 32 or 64 heads per
 * workgroup: every phase of its one or two 64-row super-tiles runs on all
 * eight waves, for the latency-bound low-batch regime (vLLM PR #52212 page,
 * motivation and implementation item 2).  The pipelined kernel streams
 * longer splits in 32-row tiles. */
#define DSV4_KERNEL_PIPELINED 0
#define DSV4_KERNEL_SHORT 1

/* Plan a decode without launching anything: validates the descriptor
 * (pointers other than workspace are not looked at) and picks the head
 * grouping and the split count.  Heads per workgroup (a multiple of 16 that
 * divides H, at most 64), with S chosen for each candidate grouping as
 * below: when the selector chooses S, the smallest grouping whose S >= 2
 * fills the chip (one more split would take B * (want + 1) * head_groups
 * past 256 workgroups, one per compute unit) with at most 8 tiles of 32
 * entries per split; otherwise the largest grouping that fills the chip,
 * else 16 (with a forced S: B * S * head_groups >= 256).  num_splits = 0
 * lets the selector choose:
 *   B >= 256                 -> 1 (one workgroup per token already fills the
 *                               chip; SGLang PR #26383 page, implementation
 *                               item 3: no split-K at >= 256 tokens);
 *   otherwise want = clamp(floor(256 / (B * head_groups)), 1,
 *   min(32, T)) with T = ceil((topk+swa)/32) tiles (32: the vLLM PR #52212
 *   page, implementation item 2, cap for long context at low batch; its
 *   cap of 4 for short work is not applied, as more splits measured faster
 *   here), and S = ceil(T / ceil(T / want)): the fewest splits with the
 *   same whole tiles per split, so none is left without entries.
 * A forced num_splits must lie in [1, DSV4_MAX_SPLITS]. */
int dsv4_sparse_decode_plan(const dsv4_decode_desc* desc, int32_t num_splits, dsv4_plan* plan);

/* Scratch bytes a decode with this descriptor and split request needs
 * (0 when S = 1).  Returns 0 also for an invalid descriptor. */
size_t dsv4_sparse_decode_workspace_bytes(const dsv4_decode_desc* desc, int32_t num_splits);

/* Sparse FP8 MLA decode with an attention sink.
 *
 * Query token b belongs to sequence r = b / s_q (s_q = tokens_per_seq, 1
 * when 0): the s_q tokens of a sequence (multi-token / MTP decode) each
 * have their own q and topk_idx rows and share the sequence's block-table
 * row and valid_len entry.  (SGLang PR #26208 report, gather+dequant
 * kernel: the top-k length of token t is read at t // s_q.)
 * For token b and head h, entry k of topk_idx row b (columns [0, topk) are
 * the main list, [topk, topk+swa) the sliding window) takes part iff
 *   idx = topk_idx[b, k] >= 0, and
 *   k >= topk, or valid_len is NULL, or k < clamp(valid_len[r], 0, topk), and
 *   its page resolves: with a block table, idx/block_size <
 *   max_blocks_per_seq and page = block_table[r, idx/block_size] lies in
 *   [0, num_blocks); without one (block_table NULL), idx is a pool slot and
 *   page = idx/block_size must be < num_blocks.  The offset is idx%block_size.
 * With v_k the dequantised 512-wide row and s_k = sm_scale * q[b,h,:].v_k:
 *   out[b,h,:] = sum_k e^{s_k - lse} v_k,
 *   lse[b,h]   = ln(sum_k e^{s_k} + e^{sink[h]})   (natural log; the sink
 *                term is absent when sink is NULL).
 * A (b,h) with no taking-part entry gets out = 0 and lse = sink[h], or
 * -inf without a sink.  Entries are counted as a multiset (duplicates
 * count twice).  (vLLM PR #52212 page, implementation item 1: one 512-wide
 * QK dot over NoPE+RoPE, masked tail, attention sink and invalid-index
 * semantics; SGLang PR #26208 report, gather+dequant kernel: -1 is invalid
 * and entries at or past the top-k length are masked; unified kernel:
 * output and LSE with an attention sink.)
 *
 * Arguments (all device pointers, caller-owned):
 *   q          bf16 [B, H, 512], contiguous, 16-byte aligned; q[...,j]
 *              pairs with row dim j (448 NoPE then 64 RoPE)
 *   kv_cache   uint8 [num_blocks, page_stride], 8-byte aligned
 *   block_table int32 [B / s_q, block_table_stride] or NULL
 *   topk_idx   int32 [B, topk_idx_stride], columns [0, topk+swa) used
 *   valid_len  int32 [B / s_q] or NULL
 *   sink       float [H] or NULL
 *   out        bf16 [B, H, 512], contiguous, 16-byte aligned
 *   lse        float [B, H] or NULL (not written)
 *   num_splits 0 = selector, else the split count to use
 * The split count changes results only by rounding; with S > 1 the call
 * needs desc->workspace of at least dsv4_sparse_decode_workspace_bytes().
 * Launches the partial kernel and, when S > 1, the combine kernel. */
int dsv4_sparse_decode(const dsv4_decode_desc* desc, const void* q, const void* kv_cache,
                       const int32_t* block_table, const int32_t* topk_idx,
                       const int32_t* valid_len, const float* sink, void* out, float* lse,
                       int32_t num_splits, hipStream_t stream);

/* dsv4_sparse_decode through a block table that also writes the req-local
 * -> global conversion of the same indices, so that a decode step which
 * needs both the attention output and the global slots (later consumers of
 * the slots) reads the indices and the table once.
 * (vLLM PR #52212 page, implementation item 1: the decode resolves entries
 * through the block table; vLLM PR #41217 report, key source snippets: the
 * req-index to global-index conversion.)
 *   block_table   required (int32 [B / s_q, block_table_stride])
 *   global_slots  int32 [B, topk + swa], contiguous, 4-byte aligned, device:
 *                 exactly what dsv4_convert_req_index_to_global writes for
 *                 topk_idx with req_id[t] = t / s_q, num_reqs = B / s_q,
 *                 width = topk + swa, ti_stride = topk_idx_stride,
 *                 max_blocks_per_req = desc->max_blocks_per_seq, no
 *                 cu_seqlens and invalid_fill = -1.  Every column is
 *                 converted, the masked tail [valid_len, topk) included.
 * out and lse are the bytes dsv4_sparse_decode writes for the same
 * arguments.  The partial kernel writes the slots from index and table
 * loads issued beside its own: the short-split kernel always, the
 * pipelined kernel when a split covers at most 1024 index columns
 * (ceil((topk + swa) / S) <= 1024); otherwise a conversion launch precedes
 * the decode on the same stream.  Errors as dsv4_sparse_decode, plus
 * INVALID_ARGUMENT for a NULL block_table or global_slots or a misaligned
 * global_slots (nothing launched). */
int dsv4_sparse_decode_with_slots(const dsv4_decode_desc* desc, const void* q,
                                  const void* kv_cache, const int32_t* block_table,
                                  const int32_t* topk_idx, const int32_t* valid_len,
                                  const float* sink, void* out, float* lse, int32_t num_splits,
                                  int32_t* global_slots, hipStream_t stream);

/* First stage of dsv4_sparse_decode_with_slots alone: the split partials (or,
 * with S = 1, out and lse) exactly as dsv4_sparse_decode_partial writes
 * them, and the global slots exactly as dsv4_sparse_decode_with_slots
 * writes them.  Same arguments and errors as dsv4_sparse_decode_with_slots. */
int dsv4_sparse_decode_partial_with_slots(const dsv4_decode_desc* desc, const void* q,
                                          const void* kv_cache, const int32_t* block_table,
                                          const int32_t* topk_idx, const int32_t* valid_len,
                                          const float* sink, void* out, float* lse,
                                          int32_t num_splits, int32_t* global_slots,
                                          hipStream_t stream);

/* First stage of dsv4_sparse_decode alone.  With S = 1 it writes out/lse
 * directly (the same bytes dsv4_sparse_decode writes).  With S > 1 it
 * writes, for every (b, h, split), the split's normalised partial output
 * and its log-sum-exp without the sink, into the workspace:
 *   part_out = (bf16*)workspace                       bf16 [B, H, S, 512] (RNE)
 *   part_lse = (float*)(part_out + B*H*S*512)         float [B, H, S]
 * (B*H*S*1028 bytes in all).
 * A split with no taking-part entry writes 0 and -inf.  Splits cover the
 * row's effective list main[0:valid_len] ++ swa in contiguous chunks
 * (vLLM PR #52212 page, implementation item 2: per-row active splits under
 * a fixed grid). */
int dsv4_sparse_decode_partial(const dsv4_decode_desc* desc, const void* q,
                               const void* kv_cache, const int32_t* block_table,
                               const int32_t* topk_idx, const int32_t* valid_len,
                               const float* sink, void* out, float* lse, int32_t num_splits,
                               hipStream_t stream);

/* Merge S split partials with the sink by log-sum-exp:
 *   M = max(max_s part_lse[b,h,s], sink[h]),
 *   D = sum_s e^{part_lse - M} + e^{sink[h] - M},
 *   out[b,h,:] = sum_s e^{part_lse - M} part_out[b,h,s,:] / D  (bf16, RNE),
 *   lse[b,h] = M + ln D.
 * All splits empty: out = 0, lse = sink[h] (or -inf without a sink).  A
 * split with part_lse = -inf adds nothing, whatever its part_out row holds.
 * For a given S the result is deterministic; the launch shape (and with it
 * the order in which splits are added) depends on B*H and S, so results for
 * different B*H may differ in the last bf16 bit.
 * (SGLang PR #26208 report, implementation item 3: split-K over the top-k
 * axis; vLLM PR #52212 page: the reduce of split partials.)
 *   part_out bf16 [B, H, S, 512] (8-byte aligned), part_lse float [B, H, S],
 *   sink float [H] or NULL, out bf16 [B, H, 512], lse float [B, H] or NULL.
 * Also serves partials computed elsewhere (e.g. on other GPUs). */
int dsv4_combine_splits(int32_t batch, int32_t num_heads, int32_t num_splits,
                        const void* part_out, const float* part_lse, const float* sink,
                        void* out, float* lse, hipStream_t stream);

/* ----------------------------------------------- allocation-free decode */

/* Bytes of the library's own split-partial scratch (32 MiB per GPU). */
#define DSV4_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* dsv4_sparse_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, but with S > 1 the split
 * partials go to a fixed device array inside this library instead of
 * desc->workspace, which is ignored.
 *   - The array holds DSV4_NOALLOC_SCRATCH_BYTES; a call whose partials
 *     (dsv4_sparse_decode_workspace_bytes) would not fit returns
 *     DSV4_ERR_WORKSPACE_TOO_SMALL and launches nothing.
 *   - Each GPU has its own array, loaded with the library's code and kept
 *     until the process ends.  Its device address is looked up on the first
 *     call made with that GPU current; stream must belong to the current
 *     GPU (DSV4_ERR_INVALID_ARGUMENT otherwise).
 *   - All calls on one GPU share its array, which keeps the last call's
 *     partials: calls that overlap on one GPU (other streams, other
 *     threads) race and give undefined results.  Calls ordered on one
 *     stream are safe.
 *   - Nothing is allocated or freed; the call never synchronises.
 * Arguments and everything else as for dsv4_sparse_decode. */
int dsv4_sparse_decode_noalloc(const dsv4_decode_desc* desc, const void* q, const void* kv_cache,
                               const int32_t* block_table, const int32_t* topk_idx,
                               const int32_t* valid_len, const float* sink, void* out, float* lse,
                               int32_t num_splits, hipStream_t stream);

/* ---------------------------------------------------------- dual cache */

/* One fp8_ds_mla pool: its pages and how a sequence's req-local slots map
 * onto them (geometry as in dsv4_decode_desc). */
typedef struct dsv4_cache_pool {
    const void* kv_cache;          /* uint8 [num_blocks, page_stride], 8-byte aligned */
    const int32_t* block_table;    /* int32 [B / s_q, block_table_stride] or NULL     */
    int64_t num_blocks;            /* >= 1                                            */
    int64_t page_stride;           /* multiple of 8, >= block_size * 584              */
    int64_t block_table_stride;    /* elements between block-table rows               */
    int32_t block_size;            /* slots per page, >= 1                            */
    int32_t max_blocks_per_seq;    /* usable block-table columns                      */
} dsv4_cache_pool;

/* Dual-cache decode: as dsv4_sparse_decode, except that main entries
 * (columns [0, topk)) resolve in main_pool and sliding-window entries
 * (columns [topk, topk+swa)) in swa_pool, each through its own block table,
 * block size and page stride.  The cache geometry fields of desc are
 * ignored (the pools carry it); both pools have a block table or neither
 * does.  (vLLM PR #52212 page: main/SWA work in one kernel, implementation
 * item 1, next to a separate compressed "extra" cache, item 3; DeepSeek-V4
 * keeps its sliding-window cache apart from that cache.) */
int dsv4_sparse_decode_dual(const dsv4_decode_desc* desc, const void* q,
                            const dsv4_cache_pool* main_pool, const dsv4_cache_pool* swa_pool,
                            const int32_t* topk_idx, const int32_t* valid_len, const float* sink,
                            void* out, float* lse, int32_t num_splits, hipStream_t stream);

/* -------------------------------------------------- two-kernel path */

/* The two-kernel decode: gather + dequantise into a dense bf16 buffer, then
 * attention over it.  Results equal dsv4_sparse_decode's up to rounding (the
 * same bf16 rows enter the same products); the fused call moves about 2.7x
 * fewer bytes and is the production path.  (SGLang PR #26208 report: the
 * gather+dequant kernel writing bf16 KV plus a mask, then the unified sparse
 * attention kernel over it; SGLang PR #26383 page, implementation item 3:
 * the fused kernel against this separate path.)
 *
 * Stage 1.  For every token b and column k of its topk_idx row, writes the
 * dequantised row (448 NoPE then 64 RoPE values, bf16) to
 * kv_out[b, k, :] and mask_out[b, k] = 0 when the entry takes part under
 * the rules of dsv4_sparse_decode, else 1 with a zero row.  desc->flags may
 * hold DSV4_DECODE_SCRUB (non-finite elements written as 0).
 *   kv_out   bf16 [B, topk+swa, 512], 16-byte aligned
 *   mask_out uint8 [B, topk+swa]
 * Other arguments as for dsv4_sparse_decode (q and sink are not needed). */
int dsv4_gather_dequant(const dsv4_decode_desc* desc, const void* kv_cache,
                        const int32_t* block_table, const int32_t* topk_idx,
                        const int32_t* valid_len, void* kv_out, uint8_t* mask_out,
                        hipStream_t stream);

/* Stage 2.  Attention with the sink over kv_dense [B, topk+swa, 512] bf16
 * (16-byte aligned) where entry k of token b takes part iff mask[b, k] == 0;
 * out, lse, num_splits and the workspace as for dsv4_sparse_decode (the
 * splits cover all topk+swa entries).  Only batch, num_heads, topk, swa,
 * sm_scale and the workspace fields of desc are used (the cache geometry
 * must still be valid); desc->flags must be 0. */
int dsv4_dense_decode(const dsv4_decode_desc* desc, const void* q, const void* kv_dense,
                      const uint8_t* mask, const float* sink, void* out, float* lse,
                      int32_t num_splits, hipStream_t stream);

/* ------------------------------------------------------ cache writer */

/* Store flag: sanitise while quantising (see dsv4_quantize_store). */
#define DSV4_STORE_SANITIZE 0x1u

/* Quantise bf16 rows and store them into the fp8_ds_mla cache.
 *
 * Row i (512 bf16: dims [0, 448) NoPE, [448, 512) RoPE) goes to global slot
 * s = slot_mapping[i]: row s % block_size of page s / block_size, in the
 * page layout above.  For NoPE group g (dims [64g, 64g+64)) let a be the
 * largest |x| of the group, NaN elements left out; its UE8M0 code is the
 * smallest c in [0, cap] with a <= 448 * 2^(c-127) (cap when none is, i.e.
 * for an infinity), and each element is stored as the E4M3FN rounding
 * (nearest, ties to even) of x * 2^(127-c) clamped to [-448, 448]; a NaN
 * element stores 0x7F.  RoPE values are stored bit for bit.  Scale byte 7
 * is 0.  With DSV4_STORE_SANITIZE, cap = 254 and a NaN or infinite RoPE
 * value is stored as +0, so that a cache written from finite NoPE inputs
 * holds no non-finite value and decodes without DSV4_DECODE_SCRUB;
 * without it cap = 255 (a NaN scale).  (vLLM PR #52212 page, the sanitising
 * writer snippet: code clamp [0, 254] vs [0, 255], RoPE non-finite -> 0.
 * The amax -> code rule is not printed there; the smallest sufficient code
 * is the reading taken.)
 *
 * Arguments (device pointers, caller-owned):
 *   rows          bf16 [num_rows, row_stride], 16-byte aligned,
 *                 row_stride a multiple of 8 and >= 512
 *   slot_mapping  int64 [num_rows]; a negative slot or one past the pool
 *                 (s / block_size >= num_blocks) skips its row
 *   kv_cache      uint8 [num_blocks, page_stride], 8-byte aligned,
 *                 page_stride a multiple of 8 and >= block_size * 584
 *   flags         0 or DSV4_STORE_SANITIZE
 * Only the 576 data bytes and 8 scale bytes of each stored row are
 * written.  Slots must be distinct: rows sharing a slot race, and the bytes
 * left there are unspecified.  num_rows = 0 launches nothing. */
int dsv4_quantize_store(const void* rows, int64_t row_stride, const int64_t* slot_mapping,
                        int64_t num_rows, void* kv_cache, int32_t block_size, int64_t num_blocks,
                        int64_t page_stride, uint32_t flags, hipStream_t stream);

/* ------------------------------------------------- index conversion */

/* Req-local -> global slot conversion through a block table.  For token t
 * (request r = req_id[t], or t when req_id is NULL) and column i:
 *   idx = token_indices[t*ti_stride + i];
 *   fill when idx < 0, r outside [0, num_reqs), idx/block_size >=
 *   max_blocks_per_req, page = block_table[r*bt_stride + idx/block_size] < 0,
 *   or page*block_size + idx%block_size > INT32_MAX (computed in 64 bits);
 *   otherwise page*block_size + idx%block_size.
 * Dense (cu_seqlens NULL): out[t*width + i] for i < width.
 * Ragged: out[cu_seqlens[t] + i] for i < min(cu_seqlens[t+1]-cu_seqlens[t],
 * width) and inside [0, cu_seqlens[num_tokens]); nothing else is written.  invalid_fill = 0 reproduces the page's
 * kernel; -1 feeds dsv4_sparse_decode with block_table = NULL.
 * (vLLM PR #41217 report, key source snippets: the req-index to
 * global-index kernel, its ragged store from seq_start and block range
 * check.)  Bit-exact integer work.
 *   req_id int32 [num_tokens] or NULL; block_table int32 [num_reqs, bt_stride];
 *   token_indices int32 [num_tokens, ti_stride]; cu_seqlens int32
 *   [num_tokens+1] or NULL; out int32 as above. */
int dsv4_convert_req_index_to_global(const int32_t* req_id, int32_t num_reqs,
                                     const int32_t* block_table, int64_t bt_stride,
                                     int32_t max_blocks_per_req, const int32_t* token_indices,
                                     int64_t ti_stride, int32_t num_tokens, int32_t width,
                                     int32_t block_size, const int32_t* cu_seqlens,
                                     int32_t invalid_fill, int32_t* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DSV4_H */
