/*
 * nsa_compress.h - C ABI of the NSA KV-compression operator
 * (NsaCompressWithCache), built into the same library as compressor.h.
 *
 * Page cited: [NSA] the aclnnNsaCompressWithCache article (功能说明与压缩算法流程,
 * 计算公式, 参数说明, 约束说明).  Status codes are the CMP_* codes of
 * compressor.h.  All pointers are HIP device addresses on the current
 * device unless marked (host); the library allocates nothing and never
 * synchronises: the work is enqueued on `stream`.
 */
#ifndef NSA_COMPRESS_H
#define NSA_COMPRESS_H

#include <stddef.h>
#include <stdint.h>

#include "compressor.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { NSA_BF16 = 0, NSA_F16 = 1 };                 /* dtype of input, weight and cache */
enum { NSA_LAYOUT_PAGED = 0, NSA_LAYOUT_TND = 1 };  /* how input holds the tokens */

/* Device error bits OR-ed into *device_error (the batch concerned writes
 * nothing; no out-of-range access happens). */
#define NSA_DEVERR_SLOT 1u    /* slotMapping[b] outside [0, result_len) */
#define NSA_DEVERR_TABLE 2u   /* a block-table entry outside [0, num_blocks), or
                                 the window beyond table_stride blocks */
#define NSA_DEVERR_SEQLEN 4u  /* act_seq_len[b] < 0, or (packed) rows beyond T */

/* Static shape ([NSA] 约束说明).
 * head_num             N: 1..64, even when above 50.
 * head_dim             D: a multiple of 16, at most 256.
 * compress_block_size  window of tokens compressed into one: a multiple of 16,
 *                      at least compress_stride, at most 64.
 * compress_stride      16, 32, 48 or 64.
 * page_block_size      64 or 128 (paged layout).
 * dtype                NSA_BF16 or NSA_F16.
 * layout               NSA_LAYOUT_PAGED (input [num_blocks, page_block_size,
 *                      N, D] with a block table) or NSA_LAYOUT_TND (input
 *                      [T, N, D], the batches' tokens packed in batch order).
 * Any other value is CMP_ERR_UNSUPPORTED (or CMP_ERR_INVALID for sizes). */
typedef struct nsa_shape {
  int32_t head_num;
  int32_t head_dim;
  int32_t compress_block_size;
  int32_t compress_stride;
  int32_t page_block_size;
  int32_t dtype;
  int32_t layout;
} nsa_shape;

/* Arguments of one call.
 * input          (device) the KV cache, layout as above, read only.
 * weight         (device) [compress_block_size, N]: column n weights head n.
 * slot_mapping   (device) int32 [batch]: output row of batch b's compressed
 *                token; values must be distinct.
 * act_seq_len    (device) int64 [batch]: each batch's current length s
 *                (actSeqLenType 1 of the page).
 * block_table    (device) int32 [batch, table_stride] (paged layout; NULL
 *                for TND): block of token t of batch b is
 *                block_table[b, t / page_block_size].
 * batch          number of batches (>= 1).
 * table_stride   entries per block-table row (paged).
 * num_blocks     blocks of input (paged).
 * T              rows of input (TND).
 * output_cache   (device) [result_len, N, D], updated in place: only the
 *                rows of compressing batches change.
 * result_len     rows of output_cache.
 * device_error   (device) uint32 word the kernel ORs NSA_DEVERR_* bits into
 *                (the caller clears it); may be NULL. */
typedef struct nsa_args {
  const void* input;
  const void* weight;
  const int32_t* slot_mapping;
  const int64_t* act_seq_len;
  const int32_t* block_table;
  int32_t batch;
  int32_t table_stride;
  int32_t num_blocks;
  int64_t T;
  void* output_cache;
  int64_t result_len;
  uint32_t* device_error;
} nsa_args;

/* One NsaCompressWithCache call ([NSA] 算法流程, 计算公式): every batch b with
 * s = act_seq_len[b] >= compress_block_size and (s - compress_block_size) %
 * compress_stride == 0 writes, to output_cache[slot_mapping[b]], the sum over
 * its last compress_block_size tokens of token[j][n][d] * weight[j][n],
 * accumulated in fp32 in token order and rounded nearest-even to the dtype.
 * Other batches write nothing.  Returns CMP_OK or a CMP_ERR_* code (checked
 * on the host before any launch). */
int nsa_compress_with_cache(const nsa_shape* shape, const nsa_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NSA_COMPRESS_H */
