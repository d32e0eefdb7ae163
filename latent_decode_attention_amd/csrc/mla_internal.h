// Internal interface between the host-side planner (mla_api.cpp) and the
// device kernels (mla_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "mla_fastdiv.h"

namespace mla {

constexpr int kDqk = 576;        // latent row width: kv_lora_rank 512 + RoPE 64
constexpr int kDv = 512;         // value columns = leading kv_lora_rank columns
constexpr int kTile = 64;        // tokens staged in LDS per pipeline step
constexpr int kMaxRowsPerGroup = 128;  // query rows (q token x head) per work-group: 128 or 64
constexpr int kMaxHeads = 128;         // query heads per token
constexpr int kMaxQPerGroup = 4;       // query tokens per work-group (attended masks kept per token)

// Everything one decode launch needs.  Passed by value as the kernel argument.
struct DecodeArgs {
  const uint16_t *q;           // bf16 [B, Q, h_q, 576]
  const uint16_t *kv;          // bf16 [num_blocks, block_size, 576], or int8 when kv8
  const int32_t *block_table;  // [B, max_blocks]
  const int32_t *seq_lens;     // [B]
  const int32_t *indices;      // sparse only
  int64_t idx_stride_b, idx_stride_q;
  int32_t top_k;
  // Sparse under DCP (own_lists non-null): each work-group picks its shard's
  // valid entries out of its unit's list, in list order, and keeps the ones
  // of its partition at own_lists[unit * top_k + i] (i = the entry's rank among
  // the shard's); by_interleave and by_shards divide a position into its
  // shard.  Null otherwise.
  int32_t *own_lists;
  FastDiv by_interleave, by_shards;
  int32_t sparse;
  int32_t B, Q, h_q;
  int32_t block_size, bs_shift, max_blocks, num_blocks;
  float scale_log2;            // scale * log2(e): scores are kept in base-2 units
  int32_t num_shards, interleave, shard_base, shard_units;
  int32_t q_per_group, rows_per_group, q_groups;
  int32_t head_chunks;         // groups per query token (heads cut into chunks of rows_per_group), else 1
  int32_t kernel_rows;         // work-group shape: 128 or 64 query rows (>= rows_per_group)
  int32_t splits, chunk;
  int64_t rows_total;          // B * Q * h_q
  // final results (splits == 1)
  void *out;
  int32_t out_fp32;
  float *lse;
  // split-KV partial results (splits > 1): O [shard_units * splits, rows_total, 512] as fp32,
  // or (part_f16) as fp16 scaled per (row, 128-column quarter) with the inverse scales in
  // part_scale [shard_units * splits, rows_total, 4]; lse [shard_units * splits, rows_total]
  void *part_o;
  float *part_lse;
  float *part_scale;
  int32_t part_f16;
  // int8 cache (kv8): `kv` holds int8 rows and kv_scale fp32 [num_blocks, block_size] their factors
  int32_t kv8;
  const float *kv_scale;
};

struct MergeArgs {
  const void *o_parts;    // [groups * n, rows, d_v], fp32, or fp16 when f16
  const float *lse_parts; // [groups * n, rows]
  const float *scale_parts;  // f16 only: [groups * n, rows, d_v / 128] inverse scales
  int32_t f16;
  int32_t n;
  int64_t rows;
  int32_t d_v;
  int32_t groups;
  void *out;              // [groups, rows, d_v]
  int32_t out_fp32;
  float *lse_out;         // [groups, rows]
};

// Latent KV-cache write through a slot map (optionally one DCP shard's tokens).
struct KvWriteArgs {
  const void *rows;            // bf16 [T, 576]
  const int32_t *slots;        // [T]
  int64_t T;
  void *kv;                    // bf16 [num_slots, 576]
  int64_t num_slots;
  const int32_t *positions;    // [T], read only when num_shards > 1
  int32_t num_shards, interleave, shard_id;
};

// Top-k selection over indexer scores: row (b, q) holds the scores of positions
// [0, L) with L = clamp(seq_lens[b] - Q + q + 1, 0, max_len) at
// scores[b * stride_b + q * stride_q + p]; out [B, Q, top_k] receives the
// selected positions in ascending order, -1 padded.
struct TopkArgs {
  const float *scores;
  int64_t stride_b, stride_q;
  const int32_t *seq_lens;
  int32_t B, Q, max_len, top_k;
  int32_t *out;
};

// Enqueue the kernels; return the HIP status of the launch.
hipError_t launch_decode(const DecodeArgs &args, int64_t grid, hipStream_t stream);
hipError_t launch_topk(const TopkArgs &args, hipStream_t stream);
hipError_t launch_merge(const MergeArgs &args, hipStream_t stream);
hipError_t launch_kv_write(const KvWriteArgs &args, hipStream_t stream);

// Device scratch for the entry point that allocates nothing: a fixed array in
// device memory (one per device, for the life of the process).  On success
// *ptr is its device address on the current device (looked up once per
// device) and *bytes its size.
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_buffer(void **ptr, size_t *bytes);

}  // namespace mla
