/*
 * libmla_decode — MLA decode attention over a paged latent KV cache on AMD
 * Instinct MI355X (gfx950).
 *
 * Operation (notation of "RFC: MsModeling 支持 Decode Context Parallel 仿真",
 * §2.1.4 symbol table): B sequences, Q query tokens per sequence (Q = 1 plus
 * speculative tokens), h_q query heads, one latent KV row per token shared by
 * every head (h_kv = 1 for MLA) of D = kv_lora_rank + qk_rope_head_dim = 576
 * bf16 columns, stored as [num_blocks, block_size, D] behind a block table
 * (§2.1.4.1, table A).  For sequence b of length S_b, query token q sits at
 * position pos = S_b - Q + q and attends a set A(b, q) of positions <= pos:
 *
 *   row(b, p) = block_table[b, p / block_size] * block_size + p % block_size
 *   s_p       = scale * <q[b, q, h, 0:576], kv[row(b, p), 0:576]>
 *   lse       = ln sum_{p in A} exp(s_p)                      (fp32)
 *   out       = sum_{p in A} exp(s_p - lse) * kv[row(b, p), 0:512]
 *
 * V is the first d_v = 512 (kv_lora_rank) columns of the same latent row, and
 * the output stays in that latent space (the up-projection is applied by the
 * caller).  An empty A gives out = 0 and lse = -inf.  The attention op returns
 * the fp32 lse next to the output as the DCP page's table B asks
 * (§2.1.4.2, softmax_lse_flag).
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are HIP device pointers; the library reads and
 *    writes them only from kernels enqueued on `stream` (a hipStream_t; NULL
 *    is the null stream).  The caller owns every buffer.  The library never
 *    allocates, frees or synchronizes, and is safe to call from several host
 *    threads (calls on one stream run in order; calls that share an output or
 *    workspace buffer on different streams race).  The only state it keeps is
 *    what it learns of each device on its first call there (the architecture,
 *    checked to be gfx950, and the compute-unit count).
 *  - Arrays are dense, row-major, with the shapes given below.
 *  - Arguments are checked on the host before anything is enqueued; a failed
 *    check returns its status and enqueues nothing (the failure rules of the
 *    DCP page §2.1.3: illegal configurations are errors, raised before the
 *    backend).  Device data (seq_lens, block_table, indices) is not inspected
 *    on the host: positions outside [0, pos], and block-table entries outside
 *    [0, num_blocks) for a position that is attended, are skipped on the device
 *    instead of being read.  Callers must keep seq_lens[b] <= max_seq_len and
 *    seq_lens[b] <= max_blocks * block_size.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
  MLA_ERR_BAD_SHAPE = 2,           /* a size or stride is out of range */
  MLA_ERR_UNSUPPORTED = 3,         /* valid but not implemented (e.g. d_qk != 576) */
  MLA_ERR_WORKSPACE_TOO_SMALL = 4, /* workspace_bytes < mla_workspace_size(...) */
  MLA_ERR_LAUNCH = 5,              /* the HIP runtime rejected a kernel launch */
  MLA_ERR_DEVICE = 6,              /* the current HIP device is missing or not a gfx950 (checked
                                      on the host once per device, before any launch) */
  MLA_ERR_SCRATCH_LIMIT = 7        /* mla_decode_sparse_noalloc: the call needs more scratch than
                                      the library's fixed buffer (MLA_NOALLOC_SCRATCH_BYTES) */
} mla_status_t;

typedef enum { MLA_DTYPE_BF16 = 0, MLA_DTYPE_FP32 = 1 } mla_dtype_t;

/* Problem description shared by the decode calls. */
typedef struct {
  int32_t B;                  /* sequences, >= 1 */
  int32_t Q;                  /* query tokens per sequence, 1..16; causal among them */
  int32_t h_q;                /* query heads, 1..128 */
  int32_t d_qk;               /* latent row width; must be 576 */
  int32_t d_v;                /* value width (leading columns of the row); must be 512 */
  float scale;                /* softmax scale applied to <q, k>: finite and > 0 */
  const void *q;              /* device, bf16 [B, Q, h_q, d_qk] (query already absorbed
                                 into the latent space; RoPE part last) */
  const void *kv;             /* device, [num_blocks, block_size, d_qk] in kv_dtype */
  int32_t num_blocks;         /* >= 1 */
  int32_t block_size;         /* tokens per block, a power of two, 1..4096 */
  const int32_t *block_table; /* device, int32 [B, max_blocks] physical block ids */
  int32_t max_blocks;         /* >= 1 */
  const int32_t *seq_lens;    /* device, int32 [B], each in [Q, max_seq_len] */
  int32_t max_seq_len;        /* host-side upper bound on every seq_lens[b]; sizes the
                                 split-KV plan, >= 1 and <= max_blocks * block_size */
  int32_t group_rows;         /* work-group shape: 0 = chosen per problem, or 64 / 128 query
                                 rows per work-group (results agree within rounding).  By
                                 default 64 is taken when the rows fit in 64 anyway, when
                                 64-row groups need no KV partitions while 128-row groups
                                 would, or when 128-row partitions would be 4 tiles or
                                 fewer.  Any other value: MLA_ERR_BAD_SHAPE */
  /*
   * Element type of the latent cache (the int8 cache is the one-byte "kv-int8"
   * element type of "RFC: MsModeling 支持 Decode Context Parallel 仿真", the notation
   * table of §2.1.4, listed again among the open items of §3.3; the pages state
   * no dequantisation rule).  MLA_KV_BF16 (0, the default of a zeroed struct): `kv` holds bf16 and
   * `kv_scale` is ignored.  MLA_KV_INT8 (1): `kv` holds int8 and `kv_scale`
   * one fp32 factor per cache row, device fp32 [num_blocks, block_size]; the
   * row's value is kv_scale[row] * kv[row, c] for all 576 columns (keys and the
   * value columns alike).  Int8 caches run with 64-row work-groups only
   * (group_rows 128 with MLA_KV_INT8: MLA_ERR_UNSUPPORTED).  A null kv_scale
   * with MLA_KV_INT8: MLA_ERR_NULL_POINTER; another kv_dtype: MLA_ERR_UNSUPPORTED.
   */
  int32_t kv_dtype;
  const float *kv_scale;
} mla_problem_t;

typedef enum { MLA_KV_BF16 = 0, MLA_KV_INT8 = 1 } mla_kv_dtype_t;

/*
 * Bytes of scratch the decode call needs for its split-KV partial results
 * (fp32 partial outputs plus their lse) and, for sparse calls under DCP, for
 * each shard's part of the index lists.  Pass the arguments the decode call
 * will get; the size is that of the very plan the call makes:
 *  num_shards, interleave, shard_id  as in mla_decode_dense / mla_decode_sparse_dcp
 *              (1, any, any for an unsharded call).  The interleave matters: the
 *              shard streams of a dense DCP call are runs of `interleave` tokens
 *              dealt round-robin ("RFC: MsModeling 支持 Decode Context Parallel
 *              仿真", §2.1.4.1), so the longest stream, and the partitions cut
 *              from it, depend on it.
 *  top_k       0 for a dense call, else the sparse call's list length.
 *  index_stride_q  the sparse call's stride between query tokens (0 = one list
 *              shared by the query tokens); ignored for dense calls.  >= 0.
 * Depends on the current HIP device's compute-unit count (256 is assumed when
 * no device is visible).  Returns 0 when the plan needs no scratch, and
 * (size_t)-1 when the arguments are invalid.  Equal to
 * mla_plan_query(...).workspace_bytes for the same arguments and num_cus.
 */
size_t mla_workspace_size(const mla_problem_t *problem, int32_t num_shards, int32_t interleave,
                          int32_t shard_id, int32_t top_k, int64_t index_stride_q);

/*
 * Dense decode: A(b, q) = { p : 0 <= p <= S_b - Q + q }.
 *
 * Decode context parallelism ("RFC: MsModeling 支持 Decode Context Parallel
 * 仿真", §1.1 and §2.1.4.1): with num_shards = N > 1 the sequence is dealt to N
 * shards in runs of `interleave` = I tokens, shard(p) = floor(p / I) mod N, and
 * shard r attends only A(b, q) ∩ { p : shard(p) = r }.  Each shard emits a
 * partial output plus lse in fp32 (the page upcasts both to fp32 before the
 * exchange, §2.1.4.3); mla_merge_lse recombines them.
 *
 *  num_shards  >= 1.  1 = unsharded; `interleave` and `shard_id` are ignored.
 *  interleave  >= 1 when num_shards > 1.
 *  shard_id    -1 = compute every shard in this call; otherwise one shard in
 *              [0, num_shards).  The two forms agree within the stated accuracy,
 *              not bit for bit: the plan (where partitions start, and so the
 *              running maxima P is rounded against) depends on the work per call.
 *  out         device.  Unsharded: [B, Q, h_q, d_v] in out_dtype.  Sharded:
 *              fp32 [n_out, B, Q, h_q, d_v] with n_out = num_shards when
 *              shard_id = -1, else 1 (out_dtype must be MLA_DTYPE_FP32).
 *  lse         device, fp32 [B, Q, h_q] (unsharded) or [n_out, B, Q, h_q].
 *  workspace   device scratch of workspace_bytes >= mla_workspace_size(problem,
 *              num_shards, interleave, shard_id, 0, 0); may be NULL when that
 *              size is 0.
 */
mla_status_t mla_decode_dense(const mla_problem_t *problem, int32_t num_shards,
                              int32_t interleave, int32_t shard_id, void *out,
                              mla_dtype_t out_dtype, float *lse, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * Sparse (DSA/SFA) decode: each query token attends only the indexer-selected
 * positions ("RFC: Context Parallel Modeling for DeepSeek-Style Attention"
 * §3.6, bf16 sparse-attention inputs; the DCP page §1.3: the sparse path
 * replaces S by top_k).  Entry (b, q, k), k < top_k, of `indices` is the
 * logical token position at indices[b * index_stride_b + q * index_stride_q + k];
 * A(b, q) is the multiset of entries i with 0 <= i <= S_b - Q + q, so -1
 * padding (anywhere in the list) and out-of-range values are dropped and a
 * repeated position counts as often as it appears.
 *
 *  indices         device, int32; the caller guarantees the strides stay inside it.
 *  top_k           list length, 1..65536.
 *  index_stride_b  elements between sequences, >= 0.
 *  index_stride_q  elements between query tokens; 0 shares one list across Q.
 *  out, lse        as the unsharded dense call.
 *  workspace       >= mla_workspace_size(problem, 1, 1, -1, top_k, index_stride_q) bytes.
 */
mla_status_t mla_decode_sparse(const mla_problem_t *problem, const int32_t *indices,
                               int32_t top_k, int64_t index_stride_b, int64_t index_stride_q,
                               void *out, mla_dtype_t out_dtype, float *lse, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * mla_decode_sparse without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, serving loops, harnesses
 * that forbid allocation).  Arguments, results and status codes as
 * mla_decode_sparse.  The call allocates nothing: the split-KV partial results
 * go to a fixed device buffer of MLA_NOALLOC_SCRATCH_BYTES that the library
 * holds on each device it runs on until the process ends (its address is
 * looked up once per device).  A call whose plan needs more scratch than that
 * (mla_workspace_size(problem, 1, 1, -1, top_k, index_stride_q) is the amount)
 * returns MLA_ERR_SCRATCH_LIMIT and enqueues nothing.  Every call on a device
 * shares that device's buffer: calls that overlap on one device (on different
 * streams, or from several host threads) race and must be serialised by the
 * caller; calls on one stream run in order.  Nothing in the buffer needs to
 * start at zero.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
mla_status_t mla_decode_sparse_noalloc(const mla_problem_t *problem, const int32_t *indices,
                                       int32_t top_k, int64_t index_stride_b, int64_t index_stride_q,
                                       void *out, mla_dtype_t out_dtype, float *lse, void *stream);

/*
 * Sparse decode under decode context parallelism: the index list of each
 * (b, q) is the globally selected top-k, and DCP rank r attends the listed
 * positions it holds, floor(i / interleave) mod num_shards == r (the
 * interleaved placement of "RFC: MsModeling 支持 Decode Context Parallel 仿真",
 * §2.1.4.1; sparse attention combined with DCP is that page's follow-up work,
 * §3.3).  Each shard emits its fp32 (O, lse) partial, which mla_merge_lse
 * combines exactly as for dense DCP; a shard that holds none of a row's
 * positions gives O = 0, lse = -inf for that row.
 *
 *  problem, indices, top_k, index_stride_b, index_stride_q  as mla_decode_sparse.
 *  num_shards  2..4096;  interleave >= 1;  shard_id in [0, num_shards) for one
 *              shard, or -1 for all shards in one call.
 *  out         device, fp32 [n_out, B, Q, h_q, 512], n_out = num_shards if
 *              shard_id = -1, else 1;  lse  device, fp32 [n_out, B, Q, h_q].
 *  workspace   >= mla_workspace_size(problem, num_shards, interleave, shard_id, top_k,
 *              index_stride_q) bytes (never 0: it holds each shard's part of
 *              every list).
 *
 * Each work-group first picks its shard's entries of its list (in list order)
 * into the workspace, then streams only those; partitions are cut for an even
 * share, min(top_k, max_seq_len) / num_shards entries, so lists that crowd one
 * shard stay correct but run longer.
 */
mla_status_t mla_decode_sparse_dcp(const mla_problem_t *problem, const int32_t *indices,
                                   int32_t top_k, int64_t index_stride_b, int64_t index_stride_q,
                                   int32_t num_shards, int32_t interleave, int32_t shard_id,
                                   float *out, float *lse, void *workspace, size_t workspace_bytes,
                                   void *stream);

/*
 * Online-softmax merge of n partial results ("RFC: MsModeling 支持 Decode
 * Context Parallel 仿真", §1.1 and §2.1.4.3: after the exchange the partial
 * outputs and lse are recombined locally).  For every row r:
 *   M = max_i lse_i;  w_i = exp(lse_i - M);  lse = M + ln sum_i w_i;
 *   out = sum_i w_i * o_i / sum_i w_i.
 * Parts with lse = -inf carry no weight; a row whose parts are all -inf gives
 * out = 0 and lse = -inf.
 *
 *  o_parts    device, fp32 [n, rows, d_v]
 *  lse_parts  device, fp32 [n, rows]
 *  n          1..1024;  rows >= 0;  d_v a multiple of 4 in 4..4096
 *  out        device, [rows, d_v] in out_dtype;  lse_out device, fp32 [rows]
 */
mla_status_t mla_merge_lse(const float *o_parts, const float *lse_parts, int32_t n,
                           int64_t rows, int32_t d_v, void *out, mla_dtype_t out_dtype,
                           float *lse_out, void *stream);

/*
 * Latent KV-cache write: the step before attention that stores the new tokens'
 * latent rows into the paged cache through a slot map ("RFC: MsModeling 支持
 * Decode Context Parallel 仿真", §2.1.4.1, table A: the MLA cache
 * [N_blk, block_size, kv_lora_rank + qk_rope_head_dim] and the int32
 * slot_mapping [total_num_tokens]; under DCP the physical cache and the slot
 * map keep their shapes and tokens are routed to ranks by interleaving at
 * cp_kv_cache_interleave_size).  For every token t:
 *
 *   if slot_mapping[t] in [0, num_slots) and (num_shards == 1 or
 *      floor(positions[t] / interleave) mod num_shards == shard_id):
 *     kv[slot_mapping[t], 0:576] = rows[t, 0:576]      (a bitwise copy)
 *
 * A negative slot marks a token this call does not store (padding, or a token
 * another rank owns); slots at or past num_slots are skipped, never written.
 * Slots stored by one call must be distinct (with a repeated slot, which of
 * the rows lands there is unspecified).  The copy moves each 1152-byte row with
 * 16-byte vector loads and stores.
 *
 *  rows          device, bf16 [T, 576], 16-byte aligned
 *  slot_mapping  device, int32 [T]
 *  T             >= 0 (0 enqueues nothing)
 *  kv            device, bf16 [num_slots, 576] (= [num_blocks, block_size, 576]),
 *                16-byte aligned; updated in place
 *  num_slots     num_blocks * block_size, >= 1
 *  positions     device, int32 [T] token positions; read only when num_shards > 1
 *  num_shards    >= 1; interleave >= 1; shard_id in [0, num_shards)
 *                (ignored when num_shards == 1)
 */
mla_status_t mla_kv_write(const void *rows, const int32_t *slot_mapping, int64_t T, void *kv,
                          int64_t num_slots, const int32_t *positions, int32_t num_shards,
                          int32_t interleave, int32_t shard_id, void *stream);

/*
 * Top-k selection of indexer scores: the positions a sparse decode attends.
 * The DSA indexer picks the 2048 best-scored positions per query token ("vllm-
 * ascend PR #18870 解读：FlashComm1 的'假开启'与 SP 归位", §4.5; "RFC: Context
 * Parallel Modeling for DeepSeek-Style Attention", §3.3 models this top-k side
 * of the fused indexer on its own); computing the scores needs the indexer's
 * trained weights and is not part of this library.
 *
 * Row (b, q) ranks positions p in [0, L) with L = min(max(seq_lens[b] - Q + q + 1,
 * 0), max_len) (query token q attends up to its own position) by the score
 * scores[b * stride_b + q * stride_q + p]: a larger score ranks higher, NaN
 * ranks below every number, -0 equals +0, and equal scores rank by position,
 * lower first.  out[b, q, 0 .. top_k) receives the min(top_k, L) best positions
 * in ascending order, then -1: directly the index list of mla_decode_sparse with
 * index_stride_b = Q * top_k and index_stride_q = top_k.  The result is unique
 * and bit-reproducible.
 *
 *  scores    device, fp32; each row readable for p < L(b, q)
 *  stride_b, stride_q  elements, >= 0
 *  seq_lens  device, int32 [B]
 *  B >= 1;  Q in 1..16;  max_len >= 1;  top_k in 1..65536
 *  out       device, int32 [B, Q, top_k]
 */
mla_status_t mla_topk_select(const float *scores, int64_t stride_b, int64_t stride_q,
                             const int32_t *seq_lens, int32_t B, int32_t Q, int32_t max_len,
                             int32_t top_k, int32_t *out, void *stream);

/* Static, human-readable name of a status. */
const char *mla_status_string(mla_status_t status);

/*
 * Host-only view of the split-KV plan a decode call would launch (no device
 * access).  `num_cus` stands in for the device's compute-unit count.
 * Returns MLA_OK and fills *plan, or the status the decode call would return
 * for these arguments.
 */
typedef struct {
  int32_t q_per_group;    /* query tokens handled together by one work-group */
  int32_t rows_per_group; /* query rows per work-group: q_per_group * h_q, or 64 when
                             h_q > 64 (each query token's heads in 64-head chunks) */
  int32_t units;          /* (sequence, query group, shard) work units */
  int32_t splits;         /* KV partitions per unit */
  int32_t chunk;          /* tokens per partition (multiple of the 64-token tile) */
  int32_t stream_len;     /* longest per-unit token stream the plan covers */
  int64_t grid;           /* work-groups in the decode launch = units * splits */
  size_t workspace_bytes; /* scratch the plan needs */
} mla_plan_t;

mla_status_t mla_plan_query(const mla_problem_t *problem, int32_t num_shards,
                            int32_t interleave, int32_t shard_id, int32_t top_k,
                            int64_t index_stride_q, int32_t num_cus, mla_plan_t *plan);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
