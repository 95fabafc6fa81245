/* Measurement aids for the sparse FP8 MLA decode library (not part of the
 * method).  Same conventions as dsv4.h: device pointers owned by the caller,
 * asynchronous on `stream`, status codes from dsv4_status, never throws. */
#ifndef DSV4_DIAG_H
#define DSV4_DIAG_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsv4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Gather floor of dsv4_sparse_decode_partial: launches the partial kernel's
 * grid (the plan for desc and num_splits) and, per workgroup, resolves the
 * same entries (index -> page through the block table, or global slots when
 * block_table is NULL) and loads the same bytes of every row (576 data bytes
 * and the 8-byte scale word; rows that take no part read a zero row), with no
 * dequantisation, no attention arithmetic and no output besides one folded
 * word per thread.  Its duration is the floor the partial kernel's memory
 * traffic sets on the same inputs.
 *   words      uint32 [plan.grid_partial * plan.block_partial] (written)
 * desc->workspace is not used.  Returns INVALID_ARGUMENT for a bad
 * descriptor or NULL kv_cache / topk_idx / words. */
int dsv4_gather_floor(const dsv4_decode_desc* desc, const void* kv_cache,
                      const int32_t* block_table, const int32_t* topk_idx,
                      const int32_t* valid_len, int32_t num_splits, uint32_t* words,
                      hipStream_t stream);

/* Phase timeline of the short-split kernel: the first stage of
 * dsv4_sparse_decode (what dsv4_sparse_decode_partial launches, same
 * results) on a plan that picks the short-split kernel, with thread 0 of
 * every workgroup recording 10 stamps into stamps[wg * 10 + k]:
 *   0  constant-rate clock (100 MHz) at entry     1  shader clock at entry
 *   2  rows resolved, loads issued (index, table) 3  super-tile 0 dequantised
 *   4  after the barrier that publishes it        5  after QK (super-tile 0)
 *   6  after the softmax (super-tile 0)           7  after the last PV
 *   8  shader clock after the output stores       9  constant-rate clock then
 * Workgroups past the plan's work units write nothing.  Returns
 * DSV4_ERR_NOT_SUPPORTED when the plan picks another kernel or the scrub flag
 * is set; otherwise as dsv4_sparse_decode_partial.
 *   stamps     uint64 [plan.grid_partial * 10] (written) */
int dsv4_short_timeline(const dsv4_decode_desc* desc, const void* q, const void* kv_cache,
                        const int32_t* block_table, const int32_t* topk_idx,
                        const int32_t* valid_len, const float* sink, void* out, float* lse,
                        int32_t num_splits, uint64_t* stamps, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSV4_DIAG_H */
