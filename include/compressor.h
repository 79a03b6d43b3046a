/*
 * compressor.h - C ABI of the MI355X (gfx950) Compressor library.
 *
 * The operator is the DeepSeek-V4 KV Compressor: every `ratio` tokens of
 * hidden states become one compressed KV row.  Definitions cited below:
 *   [PyPTO]   page "CANN PyPTO 算子实战：Compressor 长序列 KV Cache 压缩算子的原理、参数与调用方法"
 *   [CANN]    page "compressor-算子接口（torch_extension）-算子库-API参考-CANN9.2.0-beta.1开发文档"
 *   [AscendC] page "NPU DeepSeek-V4 Ascend C 融合算子优化", section Compressor
 *   [Triton]  the 10100.com article on the Triton-Ascend Compressor (CANNBot
 *             triton-op-generator)
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Pointers marked (device) are HIP device addresses on the current device;
 *   (host) are host addresses.  The caller owns every buffer; the library
 *   never allocates device memory during a call and keeps no pointer after
 *   the work it enqueued has finished.
 * - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *   Work is enqueued asynchronously; no call synchronises the host except
 *   compressor_last_device_error and compressor_timing_query.
 * - bf16 buffers hold raw bfloat16 values (2 bytes each), row-major and
 *   contiguous; fp32 and int32 likewise.
 * - Return value: a compressor_status.  Host-checkable argument errors are
 *   reported before anything is enqueued.  Value errors only visible on the
 *   device (bad table entries, negative start_pos, seqused beyond its slot,
 *   more output rows than out_rows) never cause an out-of-bounds access: the
 *   offending access is skipped and a bit is set in the workspace's error
 *   word, read with compressor_last_device_error.
 * - Calls are deterministic: no floating-point atomics, fixed reduction order
 *   ([CANN] 约束说明: deterministic computation by default).
 */
#ifndef COMPRESSOR_H_
#define COMPRESSOR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (after the aclnn NULLPTR / PARAM_INVALID / TILING_ERROR
 * convention of the NsaCompressWithCache page). */
typedef enum {
  CMP_OK = 0,
  CMP_ERR_NULLPTR = 1,      /* a required pointer is NULL */
  CMP_ERR_INVALID = 2,      /* shape or range violation */
  CMP_ERR_UNSUPPORTED = 3,  /* configuration outside the supported set */
  CMP_ERR_WORKSPACE = 4,    /* workspace_bytes below compressor_*_workspace_size */
  CMP_ERR_OUT_ROWS = 5,     /* out_rows below what the call may write */
  CMP_ERR_HIP = 6           /* a HIP runtime call failed */
} compressor_status;

/* Bits of the device error word. */
#define CMP_DEVERR_TABLE 1u      /* block-table entry outside [0, num_blocks) */
#define CMP_DEVERR_START_POS 2u  /* start_pos < 0: request treated as empty */
#define CMP_DEVERR_SEQLEN 4u     /* cu_seqlens not monotone / beyond T, seqused outside [0, slot], or
                                    more than 4 tokens in a decode request */
#define CMP_DEVERR_OUT_ROWS 8u   /* sum over requests of ceil(n_b / ratio) > out_rows */
#define CMP_DEVERR_SLOT 16u      /* compressor_epilog: slot_mapping[i] outside [-1, num_slots) */

/*
 * Static shape of a Compressor layer.
 *
 * ratio         r, tokens per compressed row: 2, 4, 8, 16, 32, 64 or 128
 *               ([CANN] 约束说明, which also names the C4A / C4Li / C128A
 *               combinations); any other value is CMP_ERR_UNSUPPORTED.  coff,
 *               the number of channel sets, is 2 for ratio 4 and 1 otherwise
 *               ([PyPTO] 参数说明).
 * head_dim      D: 128 or 512.
 * hidden        H: multiple of 512 in [1024, 10240].
 * rope_head_dim 64 (the only supported value, [PyPTO] 参数说明).
 * rotate        nonzero: multiply the result by the D x D Hadamard matrix.
 * block_size    rows per state block, 1..1024.
 * num_blocks    blocks in each state pool.
 * table_stride  int32 entries per block-table row; >= ceil(coff*r / block_size).
 */
typedef struct {
  int32_t ratio;
  int32_t head_dim;
  int32_t hidden;
  int32_t rope_head_dim;
  int32_t rotate;
  int32_t block_size;
  int32_t num_blocks;
  int32_t table_stride;
} compressor_shape;

/*
 * Arguments of one prefill or decode call.
 *
 * x                 (device) bf16 [T, H]: packed hidden states of all requests.
 * T, batch          packed rows and number of requests B (B >= 1; T == 0 is a
 *                   valid call that only zero-fills out).
 * cu_seqlens        (device) int32 [B+1] or NULL: request b's slot is rows
 *                   [cu[b], cu[b+1]) of x; NULL means B equal slots of T/B rows
 *                   (x given as [B, S, H]).  Decode requires NULL.
 * seqused           (device) int32 [B] or NULL: valid tokens of request b, the
 *                   first seqused[b] rows of its slot ([Triton] varlen packing
 *                   with cu_seqlens and seqused).  NULL: the whole slot.
 * start_pos         (device) int32 [B] or NULL: position of request b's first
 *                   token in this call; NULL means 0 ([PyPTO] 参数说明).
 * kv_state,         (device) fp32 [num_blocks, block_size, coff*D], updated in
 * score_state       place.  Request b keeps a ring of coff*r rows: position p
 *                   lives in ring slot q = p mod (coff*r), at block
 *                   table[b*table_stride + q / block_size], row q % block_size.
 *                   Rows hold all coff*D channels of kv (resp. score incl. Ape).
 *                   After a call, exactly the rows of positions
 *                   [max(s, r*floor(e/r) - (coff-1)*r), e) of this call are
 *                   stored (e = s + n); no other row changes.  Requests must
 *                   not share blocks.
 * kv_block_table    (device) int32 [B, table_stride] addressing kv_state, or
 *                   NULL to use state_block_table for both pools.
 * state_block_table (device) int32 [B, table_stride] addressing score_state.
 * w_packed          (device) bf16 [2*coff*D, H], written once per weight set by
 *                   compressor_pack_weights from wkv and wgate.
 * ape               (device) fp32 [r, coff*D]: positional bias added to the
 *                   score of position p from row p mod r.
 * norm_weight       (device) bf16 [D]: RMSNorm weight (epsilon 1e-6).
 * hadamard          (device) bf16 [D, D], required iff rotate: out = y @ hadamard.
 * sin, cos          (device) bf16 [out_rows, rope_head_dim]: row i rotates
 *                   output row i; column i drives the even element of pair i,
 *                   column rope_head_dim/2 + i the odd one.  May be NULL when
 *                   out_rows is 0.
 * out               (device) bf16 [out_rows, D]; may be NULL when out_rows is
 *                   0 (the call then only updates the state).  Request b owns rows
 *                   [o_b, o_b + ceil(n_b/r)), o_b = sum of earlier requests'
 *                   counts; its k-th completed window is row o_b + k; every
 *                   other row (windows not completed, rows past the last
 *                   request) is +0.0 ([PyPTO] 返回值说明: shape
 *                   [min(T, T//ratio + B), D], zero where nothing compresses).
 * workspace         (device) scratch of at least workspace_bytes, sized by
 *                   compressor_prefill_workspace_size / _decode_; it also holds
 *                   the device error word of the last call.  Calls sharing a
 *                   workspace must be ordered on one stream.
 */
typedef struct {
  const void* x;
  int32_t T;
  int32_t batch;
  const int32_t* cu_seqlens;
  const int32_t* seqused;
  const int32_t* start_pos;
  float* kv_state;
  float* score_state;
  const int32_t* kv_block_table;
  const int32_t* state_block_table;
  const void* w_packed;
  const float* ape;
  const void* norm_weight;
  const void* hadamard;
  const void* sin;
  const void* cos;
  void* out;
  int32_t out_rows;
  void* workspace;
  size_t workspace_bytes;
} compressor_args;

/* Workspace bytes a prefill call with T packed rows, `batch` requests and
 * out_rows output rows needs (host only, no device work). */
int compressor_prefill_workspace_size(const compressor_shape* shape, int32_t T, int32_t batch,
                                      int32_t out_rows, size_t* bytes);

/* Workspace bytes a decode call with `batch` requests (and any T <= 64)
 * needs (host only). */
int compressor_decode_workspace_size(const compressor_shape* shape, int32_t batch,
                                     int32_t out_rows, size_t* bytes);

/* Fuse wkv and wgate (device, bf16 [coff*D, H] each; [CANN] 计算公式 step 1
 * and [AscendC] 矩阵乘法: [kv, score] = X @ [W_kv, W_gate]) into one bf16
 * [2*coff*D, H] panel whose row order the kernels expect.  The panel's row
 * order is internal; only compressor_* calls read it.  Enqueued on stream. */
int compressor_pack_weights(const compressor_shape* shape, const void* wkv, const void* wgate,
                            void* w_packed, void* stream);

/* Fill both pools: kv 0, score -inf (the padding values of the first window,
 * [PyPTO] 压缩窗口与状态更新). */
int compressor_state_init(const compressor_shape* shape, float* kv_state, float* score_state,
                          void* stream);

/* Reset the ring blocks of n requests to kv 0 / score -inf.
 * kv_block_table, state_block_table  (device) int32 [table_rows, table_stride]
 *                 (kv_block_table NULL: state_block_table for both pools).
 * rows            (device) int32 [n]: table rows to reset; for each, every
 *                 block its first ceil(coff*r / block_size) entries name is
 *                 refilled (kv_state through kv_block_table, score_state
 *                 through state_block_table).  Blocks no listed row names
 *                 keep their contents.
 * table_rows      rows of the tables (>= 1 when n > 0).
 * device_error    (device) uint32 word, may be NULL: a row index outside
 *                 [0, table_rows) or a table entry outside [0, num_blocks)
 *                 is skipped (no access through it) and ORs CMP_DEVERR_TABLE
 *                 into it (the caller clears the word).
 * Returns CMP_OK (n == 0: nothing is enqueued), CMP_ERR_NULLPTR,
 * CMP_ERR_INVALID (n < 0 or table_rows < 1) or CMP_ERR_HIP. */
int compressor_state_reset(const compressor_shape* shape, float* kv_state, float* score_state,
                           const int32_t* kv_block_table, const int32_t* state_block_table,
                           const int32_t* rows, int32_t n, int32_t table_rows,
                           uint32_t* device_error, void* stream);

/* One Compressor call over packed variable-length requests ([CANN] 接口功能
 * and 计算公式; [PyPTO] 压缩窗口与状态更新; [Triton] 流式调用).  Computes the
 * fused projection, Ape, window pooling with the state rows of earlier calls,
 * RMSNorm, RoPE, the optional Hadamard product, zero rows, and the state
 * write-back described at compressor_args. */
int compressor_prefill(const compressor_shape* shape, const compressor_args* args, void* stream);

/* The same operator for decode steps of at most 4 tokens per request
 * ([Triton] 性能优化: decode has few tokens per request and different
 * scheduling; [PyPTO] 参数说明: S up to 4 for multi-token prediction).
 * x is [T, H] with T <= 64 packed rows and batch <= 64
 * (CMP_ERR_UNSUPPORTED otherwise).  cu_seqlens NULL: one row per request
 * (T == batch); else request b owns rows [cu[b], cu[b+1]).  n_b = seqused[b]
 * (or the slot length) must be <= 4: a larger value sets CMP_DEVERR_SEQLEN
 * and the request is treated as empty.  Output rows, state semantics and
 * errors are those of compressor_prefill. */
int compressor_decode(const compressor_shape* shape, const compressor_args* args, void* stream);

/* Bytes of the per-device scratch compressor_decode_noalloc uses in place of
 * a workspace; every decode call the library accepts fits. */
#define CMP_DECODE_SCRATCH_BYTES (12u << 20)

/* compressor_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels, results and limits as
 * compressor_decode, except that args->workspace and args->workspace_bytes
 * are ignored: the call works in a scratch array of CMP_DECODE_SCRATCH_BYTES
 * that the library holds on each device it runs on until the process ends.
 * No call allocates or frees anything.  Every call on a device shares that
 * device's scratch, so calls that overlap on one device (on different
 * streams, or from different threads) race and must be ordered by the
 * caller.  The scratch keeps the last call's contents; nothing in it is
 * read before the call writes it.
 * device_error  (device) uint32 word, may be NULL: the call ORs its
 *               CMP_DEVERR_* bits into it (the caller clears it);
 *               compressor_last_device_error does not apply to this entry
 *               point.
 * Returns the statuses of compressor_decode; CMP_ERR_WORKSPACE if the
 * call's layout exceeded the scratch (no accepted shape does). */
int compressor_decode_noalloc(const compressor_shape* shape, const compressor_args* args,
                              uint32_t* device_error, void* stream);

/* Quantised write of compressed rows into a paged FP8 cache, the step after
 * the operator that stores its rows into the Lightning Indexer / Sparse Flash
 * Attention compressed caches ([PyPTO] DeepSeek-V4 整网集成方式: those caches
 * may be float8).  The page gives no more than that; this entry point takes
 * the plainest reading:
 *   format     OCP FP8 E4M3 (bias 7, largest finite 448, subnormals, no
 *              infinity);
 *   scaling    one fp32 scale per 128 consecutive channels of a row:
 *              amax = max |x| of the block, scale = amax / 448, code =
 *              E4M3 round-to-nearest-even of clamp(x * (448 / amax), +-448)
 *              (fp32 arithmetic, correctly rounded); amax = 0 gives scale 0
 *              and codes +-0;
 *   placement  row i goes to cache row slot_mapping[i]; -1 writes nothing.
 * rows          (device) bf16 [n_rows, head_dim], e.g. the out rows of
 *               compressor_prefill / compressor_decode.
 * n_rows        >= 0 (0: nothing is enqueued).
 * head_dim      a multiple of 128, at most 8192 (CMP_ERR_INVALID otherwise).
 * slot_mapping  (device) int32 [n_rows]: destination row of each row, or -1.
 *               Destinations must be distinct.  A value outside
 *               [-1, num_slots) writes nothing and sets CMP_DEVERR_SLOT.
 * cache         (device) uint8 [num_slots, head_dim]: E4M3 codes, updated
 *               in place (rows not named by slot_mapping keep their bytes).
 * cache_scale   (device) fp32 [num_slots, head_dim / 128], likewise.
 * num_slots     rows of cache (>= 0).
 * device_error  (device) uint32 word the kernel ORs CMP_DEVERR_SLOT into (the
 *               caller clears it); may be NULL.
 * Returns CMP_OK, CMP_ERR_NULLPTR (a required pointer NULL with n_rows > 0),
 * CMP_ERR_INVALID or CMP_ERR_HIP (launch failure). */
int compressor_epilog(const void* rows, int32_t n_rows, int32_t head_dim,
                      const int32_t* slot_mapping, void* cache, float* cache_scale,
                      int64_t num_slots, uint32_t* device_error, void* stream);

/* Synchronise `stream`, then read the device error word (CMP_DEVERR_* bits)
 * of the last call that used `workspace` into *code. */
int compressor_last_device_error(const void* workspace, void* stream, int32_t* code);

/* Static text of a status code. */
const char* compressor_status_str(int status);

/* Row height of the prefill projection tiles for every later
 * compressor_prefill call of the process.  0 (the default): 256-row tiles
 * (8 waves per workgroup), or 128-row tiles (4 waves) when the call is too
 * short for ceil(T / 256) x (column tiles) to reach the device's compute unit
 * count, so that every unit gets work.  128 or 256 forces that height (for
 * measurement and tests; results agree within rounding, not bit for bit,
 * since the height decides which rows a tile's epilogue pools together).
 * Returns CMP_OK, or CMP_ERR_INVALID for any other value (setting unchanged).
 * Not ordered with calls already running on other threads. */
int compressor_set_prefill_tile_rows(int32_t rows);

/* Kernel timing: on = 1 brackets every kernel the library enqueues with a
 * pair of HIP events on the same stream; on = 2 only the projection GEMM
 * launches ("gemm"), for timing it inside a loop of calls with the least
 * overhead; on = 0 stops recording (other values: CMP_ERR_INVALID, with the
 * mode and the records unchanged).  Every accepted call clears the records.  Kernel names: "setup" (request plan, Hadamard check and packing,
 * staging of earlier positions' ring rows), "gemm" (projection with the window
 * pooling and state stores in its epilogue), "post",
 * "decode_main" (GEMV and ring pre-pooling),
 * "decode_tail", "pack", "state_fill", "epilog". */
int compressor_timing_enable(int32_t on);

/* Wait for the recorded events, then report the number of launches of
 * `kernel` and the sum of their durations in milliseconds. */
int compressor_timing_query(const char* kernel, int32_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* COMPRESSOR_H_ */
