// Host side of libmla_decode: argument checks, the split-KV planner and the
// C-ABI entry points declared in include/mla_decode.h.
//
// The planner sizes one launch to the device: a work-group per compute unit
// (each work-group holds two 72 KiB LDS tiles, so one fits per CU), each
// covering a query group of up to 128 or up to 64 rows.  When the natural
// units (sequence x query group x shard) are fewer than the CUs, each unit's
// token stream is cut into `splits` partitions of whole 64-token tiles; the
// partitions write partial (O, lse) pairs to the caller's workspace (fp16 O,
// scaled per row quarter, for bf16 outputs) and a merge kernel combines them
// with the same log-sum-exp rule as the DCP exchange ("RFC: MsModeling 支持
// Decode Context Parallel 仿真", §1.1, §2.1.4.3).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <atomic>
#include <mutex>

#include "../../include/mla_decode.h"
#include "mla_internal.h"

namespace {

using namespace mla;

constexpr int kDefaultCus = 256;  // MI355X
static_assert(MLA_NOALLOC_SCRATCH_BYTES == kScratchBytes, "the header states the scratch size");
constexpr int kMaxShards = 4096;
constexpr int kMaxTopK = 65536;
constexpr int kMaxMergeParts = 1024;

struct Plan {
  int q_per_group, rows_per_group, q_groups, head_chunks, shard_units;
  int kernel_rows;  // 128 or 64
  int units, splits, chunk, stream_len;
  int64_t grid;
  size_t ws_o, ws_lse, ws_scale, ws_lists, ws_total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int64_t shard_len_host(int64_t S, int64_t N, int64_t I, int64_t r) {
  if (S <= 0) return 0;
  const int64_t full = S / I, rem = S % I;
  const int64_t groups = full > r ? (full - 1 - r) / N + 1 : 0;
  return groups * I + ((full % N) == r ? rem : 0);
}

mla_status_t check_problem(const mla_problem_t *p) {
  if (!p) return MLA_ERR_NULL_POINTER;
  if (!p->q || !p->kv || !p->block_table || !p->seq_lens) return MLA_ERR_NULL_POINTER;
  if (p->d_qk != kDqk || p->d_v != kDv) return MLA_ERR_UNSUPPORTED;
  if (p->B < 1 || p->Q < 1 || p->h_q < 1 || p->num_blocks < 1 || p->max_blocks < 1 ||
      p->max_seq_len < 1)
    return MLA_ERR_BAD_SHAPE;
  if (p->Q > 16 || p->h_q > kMaxHeads) return MLA_ERR_UNSUPPORTED;
  if (p->block_size < 1 || p->block_size > 4096 || (p->block_size & (p->block_size - 1)))
    return MLA_ERR_BAD_SHAPE;
  if ((int64_t)p->num_blocks * p->block_size > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)p->max_seq_len > (int64_t)p->max_blocks * p->block_size) return MLA_ERR_BAD_SHAPE;
  if (p->max_seq_len < p->Q) return MLA_ERR_BAD_SHAPE;
  if (!std::isfinite(p->scale) || !(p->scale > 0.f)) return MLA_ERR_BAD_SHAPE;
  if (p->group_rows != 0 && p->group_rows != 64 && p->group_rows != 128) return MLA_ERR_BAD_SHAPE;
  if ((reinterpret_cast<uintptr_t>(p->q) | reinterpret_cast<uintptr_t>(p->kv)) & 15)
    return MLA_ERR_BAD_SHAPE;  // rows are moved in 16-byte pieces
  if (p->kv_dtype != MLA_KV_BF16 && p->kv_dtype != MLA_KV_INT8) return MLA_ERR_UNSUPPORTED;
  if (p->kv_dtype == MLA_KV_INT8) {
    if (!p->kv_scale) return MLA_ERR_NULL_POINTER;
    if (reinterpret_cast<uintptr_t>(p->kv_scale) & 3) return MLA_ERR_BAD_SHAPE;
    if (p->group_rows == 128) return MLA_ERR_UNSUPPORTED;  // int8 tiles leave no LDS for 128 rows
  }
  return MLA_OK;
}

mla_status_t make_plan(const mla_problem_t *p, int num_shards, int interleave, int shard_id,
                       int top_k, int64_t idx_stride_q, int num_cus, Plan *pl) {
  const bool sparse = top_k > 0;
  if (top_k < 0 || top_k > kMaxTopK) return MLA_ERR_BAD_SHAPE;
  if (num_shards < 1 || num_shards > kMaxShards) return MLA_ERR_BAD_SHAPE;
  if (num_shards > 1 && (interleave < 1 || shard_id < -1 || shard_id >= num_shards))
    return MLA_ERR_BAD_SHAPE;
  if (num_cus < 1) num_cus = kDefaultCus;
  int64_t L;
  if (sparse && num_shards > 1) {
    // Each shard streams its own part of the list (picked out by the decode
    // work-groups themselves); partitions are cut for an even share, and the
    // last partition of a unit takes whatever a skewed list adds beyond it.
    const int64_t valid = std::min<int64_t>(top_k, p->max_seq_len);
    L = (valid + num_shards - 1) / num_shards;
  } else if (sparse) {
    L = top_k;
  } else if (num_shards > 1) {
    L = 0;
    const int r0 = shard_id < 0 ? 0 : shard_id, r1 = shard_id < 0 ? num_shards : shard_id + 1;
    for (int r = r0; r < r1; ++r)
      L = std::max<int64_t>(L, shard_len_host(p->max_seq_len, num_shards, interleave, r));
  } else {
    L = p->max_seq_len;
  }
  const int64_t tiles = (L + kTile - 1) / kTile;
  const bool shared_list = !sparse || idx_stride_q == 0 || p->Q == 1;
  const int shard_units = (num_shards > 1 && shard_id < 0) ? num_shards : 1;

  // Query groups of up to R rows (R = 128 or 64) that share one token stream:
  // heads beyond R are cut into R-head chunks of one query token; fewer heads
  // are packed as whole query tokens (the most that divide Q and fit, when
  // every token of the group attends the same index list).  The token stream
  // of each (sequence, group, shard) unit is then cut into partitions until
  // the launch fills the device.
  auto layout = [&](int R, Plan *o) -> bool {
    o->kernel_rows = R;
    o->head_chunks = (p->h_q + R - 1) / R;
    o->q_per_group = 1;
    if (o->head_chunks == 1 && shared_list)
      for (int d = std::min(p->Q, kMaxQPerGroup); d > 1; --d)
        if (p->Q % d == 0 && d * p->h_q <= R) {
          o->q_per_group = d;
          break;
        }
    o->rows_per_group = o->head_chunks > 1 ? R : o->q_per_group * p->h_q;
    o->q_groups = p->Q / o->q_per_group * o->head_chunks;
    o->shard_units = shard_units;
    o->stream_len = (int)L;
    const int64_t units = (int64_t)p->B * o->q_groups * shard_units;
    if (units > INT32_MAX) return false;
    o->units = (int)units;
    int64_t max_splits = 1;
    if (units < num_cus && tiles > 1) max_splits = std::min<int64_t>((num_cus + units - 1) / units, tiles);
    // Partitions buy parallelism but their partial results must be written,
    // read back and merged.  Take the count with the lowest estimated time:
    // rounds of work-groups x (per-group fixed cost + tiles x per-tile cost),
    // plus the merge at the bytes it moves (costs measured on MI355X; sharded
    // outputs keep fp32 partials, others fp16 with 4 scales per row).
    const double t_tile = R == 128 ? 4.0 : 2.4, t_fixed = 9.0;  // microseconds
    const double part_row = num_shards > 1 ? kDv * 4.0 + 4 : kDv * 2.0 + 20;
    const double out_row = num_shards > 1 ? kDv * 4.0 + 4 : kDv * 2.0 + 4;
    const double rows = (double)p->B * p->Q * p->h_q * shard_units;
    int64_t splits = 1;
    double best = 0;
    for (int64_t s = 1; s <= max_splits; ++s) {
      const int64_t per = tiles > 0 ? (tiles + s - 1) / s : 1;
      if (tiles > 0 && (tiles + per - 1) / per != s) continue;  // same cut as fewer partitions
      const double rounds = std::ceil((double)units * s / num_cus);
      double t = rounds * (t_fixed + per * t_tile);
      if (s > 1) t += 2.0 + rows * (s * part_row + out_row) / 5.0e6;  // ~5 TB/s
      if (s == 1 || t < best) {
        best = t;
        splits = s;
      }
    }
    const int64_t tiles_per_split = tiles > 0 ? (tiles + splits - 1) / splits : 1;
    o->splits = (int)splits;
    o->chunk = (int)(tiles_per_split * kTile);
    o->grid = units * splits;
    return o->grid <= INT32_MAX;
  };
  // 128-row groups halve the per-tile fixed costs relative to the matrix
  // work; 64-row groups halve the partial results and the query rows each
  // work-group loads.  Take 64 when the groups fit in 64 rows anyway, when
  // they avoid partials altogether, or when the partitions are short enough
  // (at most 4 tiles) that the per-call costs dominate.
  Plan wide, narrow;
  if (!layout(128, &wide) || !layout(64, &narrow)) return MLA_ERR_BAD_SHAPE;
  const int64_t wide_tiles = wide.chunk / kTile;
  const int forced = p->group_rows;
  const bool use_narrow =
      p->kv_dtype == MLA_KV_INT8 ||
      (forced ? forced == 64
              : wide.rows_per_group <= 64 || (narrow.splits == 1 && wide.splits > 1) || wide_tiles <= 4);
  *pl = use_narrow ? narrow : wide;
  const int64_t splits = pl->splits;
  const int64_t rows_total = (int64_t)p->B * p->Q * p->h_q;
  if (splits > 1) {
    // Sized for fp32 partials; bf16-output calls store fp16 partials in the
    // same region plus one inverse scale per (row, 128-column quarter).
    const int64_t parts = (int64_t)pl->shard_units * splits;
    pl->ws_o = align256((size_t)(parts * rows_total * kDv) * sizeof(float));
    pl->ws_lse = align256((size_t)(parts * rows_total) * sizeof(float));
    pl->ws_scale = align256((size_t)(parts * rows_total * (kDv / 128)) * sizeof(float));
  } else {
    pl->ws_o = pl->ws_lse = pl->ws_scale = 0;
  }
  pl->ws_lists = 0;
  if (sparse && num_shards > 1) {
    // Each unit's shard entries, top_k slots per unit (its partitions fill
    // disjoint ranges of them).
    pl->ws_lists = align256((size_t)((int64_t)pl->units * top_k) * sizeof(int32_t));
  }
  pl->ws_total = pl->ws_o + pl->ws_lse + pl->ws_scale + pl->ws_lists;
  return MLA_OK;
}

// What the library learns about a device the first time a call runs on it:
// whether it is a gfx950 (the only target the kernels are built for) and its
// compute-unit count.  Looked up once per device under a lock, then read
// without one.
constexpr int kMaxDevices = 64;
struct DeviceState {
  std::atomic<int> state{0};  // 0: not looked at yet, 1: usable gfx950, -1: not usable
  int cus = kDefaultCus;
};
DeviceState g_devices[kMaxDevices];
std::mutex g_devices_mu;

// The current HIP device, if it is a usable gfx950: MLA_OK and its state.
mla_status_t current_device(DeviceState **out, int *dev_out = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  DeviceState &d = g_devices[dev];
  int st = d.state.load(std::memory_order_acquire);
  if (st == 0) {
    std::lock_guard<std::mutex> lock(g_devices_mu);
    st = d.state.load(std::memory_order_relaxed);
    if (st == 0) {
      hipDeviceProp_t prop;
      st = -1;
      if (hipGetDeviceProperties(&prop, dev) == hipSuccess && std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
          (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':')) {
        d.cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : kDefaultCus;
        st = 1;
      }
      d.state.store(st, std::memory_order_release);
    }
  }
  if (st < 0) return MLA_ERR_DEVICE;
  *out = &d;
  if (dev_out) *dev_out = dev;
  return MLA_OK;
}

// Compute units the plan is sized for: the current device's, or 256 (MI355X)
// when no usable device is visible (host-only size and plan queries).
int device_cus() {
  DeviceState *d;
  return current_device(&d) == MLA_OK ? d->cus : kDefaultCus;
}

mla_status_t run(const mla_problem_t *p, const Plan &pl, bool sparse, const int32_t *indices,
                 int top_k, int64_t stride_b, int64_t stride_q, int num_shards, int interleave,
                 int shard_id, void *out, bool out_fp32, float *lse, void *workspace,
                 size_t workspace_bytes, void *stream) {
  if (pl.ws_total > 0) {
    if (!workspace) return MLA_ERR_NULL_POINTER;
    if (workspace_bytes < pl.ws_total) return MLA_ERR_WORKSPACE_TOO_SMALL;
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return MLA_ERR_BAD_SHAPE;
  }
  if (reinterpret_cast<uintptr_t>(out) & 15) return MLA_ERR_BAD_SHAPE;
  DeviceState *dev;
  if (current_device(&dev) != MLA_OK) return MLA_ERR_DEVICE;
  DecodeArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = static_cast<const uint16_t *>(p->q);
  a.kv = static_cast<const uint16_t *>(p->kv);
  a.kv8 = p->kv_dtype == MLA_KV_INT8 ? 1 : 0;
  a.kv_scale = a.kv8 ? p->kv_scale : nullptr;
  a.block_table = p->block_table;
  a.seq_lens = p->seq_lens;
  a.indices = indices;
  a.idx_stride_b = stride_b;
  a.idx_stride_q = stride_q;
  a.top_k = top_k;
  a.sparse = sparse ? 1 : 0;
  a.B = p->B;
  a.Q = p->Q;
  a.h_q = p->h_q;
  a.block_size = p->block_size;
  a.bs_shift = 0;
  while ((1 << a.bs_shift) < p->block_size) ++a.bs_shift;
  a.max_blocks = p->max_blocks;
  a.num_blocks = p->num_blocks;
  a.scale_log2 = (float)((double)p->scale * 1.4426950408889634);
  a.num_shards = num_shards;
  a.interleave = num_shards > 1 ? interleave : 1;
  a.shard_base = (num_shards > 1 && shard_id >= 0) ? shard_id : 0;
  a.shard_units = pl.shard_units;
  a.q_per_group = pl.q_per_group;
  a.rows_per_group = pl.rows_per_group;
  a.q_groups = pl.q_groups;
  a.head_chunks = pl.head_chunks;
  a.kernel_rows = pl.kernel_rows;
  a.splits = pl.splits;
  a.chunk = pl.chunk;
  a.rows_total = (int64_t)p->B * p->Q * p->h_q;
  a.out = out;
  a.out_fp32 = out_fp32 ? 1 : 0;
  a.lse = lse;
  if (pl.splits > 1) {
    a.part_o = workspace;
    a.part_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.ws_o);
    a.part_scale = reinterpret_cast<float *>(static_cast<char *>(workspace) + pl.ws_o + pl.ws_lse);
    // bf16 results keep fp16 partials: 2^-11 relative error, a quarter of the
    // final bf16 rounding step; fp32 results keep fp32 partials.
    a.part_f16 = out_fp32 ? 0 : 1;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (sparse && num_shards > 1) {
    a.own_lists = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + pl.ws_o + pl.ws_lse + pl.ws_scale);
    a.by_interleave = make_fastdiv((uint32_t)interleave);
    a.by_shards = make_fastdiv((uint32_t)num_shards);
  }
  if (launch_decode(a, pl.grid, s) != hipSuccess) return MLA_ERR_LAUNCH;
  if (pl.splits > 1) {
    MergeArgs m;
    m.o_parts = a.part_o;
    m.lse_parts = a.part_lse;
    m.scale_parts = a.part_scale;
    m.f16 = a.part_f16;
    m.n = pl.splits;
    m.rows = a.rows_total;
    m.d_v = kDv;
    m.groups = pl.shard_units;
    m.out = out;
    m.out_fp32 = a.out_fp32;
    m.lse_out = lse;
    if (launch_merge(m, s) != hipSuccess) return MLA_ERR_LAUNCH;
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

size_t mla_workspace_size(const mla_problem_t *problem, int32_t num_shards, int32_t interleave,
                          int32_t shard_id, int32_t top_k, int64_t index_stride_q) {
  if (check_problem(problem) != MLA_OK) return (size_t)-1;
  if (index_stride_q < 0) return (size_t)-1;
  Plan pl;
  // The very plan the decode call makes for these arguments (the interleave
  // sets the longest shard stream, the list stride whether query tokens share
  // a work-group), so the size is exact.
  if (make_plan(problem, num_shards, interleave, shard_id, top_k, index_stride_q, device_cus(), &pl) != MLA_OK)
    return (size_t)-1;
  return pl.ws_total;
}

mla_status_t mla_decode_dense(const mla_problem_t *problem, int32_t num_shards,
                              int32_t interleave, int32_t shard_id, void *out,
                              mla_dtype_t out_dtype, float *lse, void *workspace,
                              size_t workspace_bytes, void *stream) {
  mla_status_t st = check_problem(problem);
  if (st != MLA_OK) return st;
  if (!out || !lse) return MLA_ERR_NULL_POINTER;
  if (out_dtype != MLA_DTYPE_BF16 && out_dtype != MLA_DTYPE_FP32) return MLA_ERR_BAD_SHAPE;
  if (num_shards > 1 && out_dtype != MLA_DTYPE_FP32) return MLA_ERR_UNSUPPORTED;
  Plan pl;
  st = make_plan(problem, num_shards, interleave, shard_id, 0, 0, device_cus(), &pl);
  if (st != MLA_OK) return st;
  return run(problem, pl, false, nullptr, 0, 0, 0, num_shards, interleave, shard_id, out,
             out_dtype == MLA_DTYPE_FP32, lse, workspace, workspace_bytes, stream);
}

mla_status_t mla_decode_sparse(const mla_problem_t *problem, const int32_t *indices,
                               int32_t top_k, int64_t index_stride_b, int64_t index_stride_q,
                               void *out, mla_dtype_t out_dtype, float *lse, void *workspace,
                               size_t workspace_bytes, void *stream) {
  mla_status_t st = check_problem(problem);
  if (st != MLA_OK) return st;
  if (!indices || !out || !lse) return MLA_ERR_NULL_POINTER;
  if (out_dtype != MLA_DTYPE_BF16 && out_dtype != MLA_DTYPE_FP32) return MLA_ERR_BAD_SHAPE;
  if (top_k < 1 || index_stride_b < 0 || index_stride_q < 0) return MLA_ERR_BAD_SHAPE;
  Plan pl;
  st = make_plan(problem, 1, 1, -1, top_k, index_stride_q, device_cus(), &pl);
  if (st != MLA_OK) return st;
  return run(problem, pl, true, indices, top_k, index_stride_b, index_stride_q, 1, 1, -1, out,
             out_dtype == MLA_DTYPE_FP32, lse, workspace, workspace_bytes, stream);
}

mla_status_t mla_decode_sparse_noalloc(const mla_problem_t *problem, const int32_t *indices,
                                       int32_t top_k, int64_t index_stride_b, int64_t index_stride_q,
                                       void *out, mla_dtype_t out_dtype, float *lse, void *stream) {
  mla_status_t st = check_problem(problem);
  if (st != MLA_OK) return st;
  if (!indices || !out || !lse) return MLA_ERR_NULL_POINTER;
  if (out_dtype != MLA_DTYPE_BF16 && out_dtype != MLA_DTYPE_FP32) return MLA_ERR_BAD_SHAPE;
  if (top_k < 1 || index_stride_b < 0 || index_stride_q < 0) return MLA_ERR_BAD_SHAPE;
  Plan pl;
  st = make_plan(problem, 1, 1, -1, top_k, index_stride_q, device_cus(), &pl);
  if (st != MLA_OK) return st;
  if (pl.ws_total > kScratchBytes) return MLA_ERR_SCRATCH_LIMIT;
  DeviceState *dev;
  if (current_device(&dev) != MLA_OK) return MLA_ERR_DEVICE;
  void *ws = nullptr;
  size_t ws_bytes = 0;
  if (pl.ws_total > 0 && scratch_buffer(&ws, &ws_bytes) != hipSuccess) return MLA_ERR_DEVICE;
  return run(problem, pl, true, indices, top_k, index_stride_b, index_stride_q, 1, 1, -1, out,
             out_dtype == MLA_DTYPE_FP32, lse, ws, ws_bytes, stream);
}

mla_status_t mla_decode_sparse_dcp(const mla_problem_t *problem, const int32_t *indices,
                                   int32_t top_k, int64_t index_stride_b, int64_t index_stride_q,
                                   int32_t num_shards, int32_t interleave, int32_t shard_id,
                                   float *out, float *lse, void *workspace, size_t workspace_bytes,
                                   void *stream) {
  mla_status_t st = check_problem(problem);
  if (st != MLA_OK) return st;
  if (!indices || !out || !lse) return MLA_ERR_NULL_POINTER;
  if (top_k < 1 || index_stride_b < 0 || index_stride_q < 0) return MLA_ERR_BAD_SHAPE;
  if (num_shards < 2) return MLA_ERR_BAD_SHAPE;
  Plan pl;
  st = make_plan(problem, num_shards, interleave, shard_id, top_k, index_stride_q, device_cus(), &pl);
  if (st != MLA_OK) return st;
  return run(problem, pl, true, indices, top_k, index_stride_b, index_stride_q, num_shards, interleave,
             shard_id, out, true, lse, workspace, workspace_bytes, stream);
}

mla_status_t mla_topk_select(const float *scores, int64_t stride_b, int64_t stride_q,
                             const int32_t *seq_lens, int32_t B, int32_t Q, int32_t max_len,
                             int32_t top_k, int32_t *out, void *stream) {
  if (!scores || !seq_lens || !out) return MLA_ERR_NULL_POINTER;
  if (B < 1 || Q < 1 || Q > 16 || max_len < 1 || top_k < 1 || top_k > kMaxTopK || stride_b < 0 ||
      stride_q < 0 || (int64_t)B * Q > INT32_MAX)
    return MLA_ERR_BAD_SHAPE;
  DeviceState *dev;
  if (current_device(&dev) != MLA_OK) return MLA_ERR_DEVICE;
  TopkArgs a;
  a.scores = scores;
  a.stride_b = stride_b;
  a.stride_q = stride_q;
  a.seq_lens = seq_lens;
  a.B = B;
  a.Q = Q;
  a.max_len = max_len;
  a.top_k = top_k;
  a.out = out;
  return launch_topk(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH;
}

mla_status_t mla_merge_lse(const float *o_parts, const float *lse_parts, int32_t n,
                           int64_t rows, int32_t d_v, void *out, mla_dtype_t out_dtype,
                           float *lse_out, void *stream) {
  if (!o_parts || !lse_parts || !out || !lse_out) return MLA_ERR_NULL_POINTER;
  if (n < 1 || n > kMaxMergeParts || rows < 0 || rows > INT32_MAX || d_v < 4 || d_v > 4096 ||
      (d_v & 3))
    return MLA_ERR_BAD_SHAPE;
  if (out_dtype != MLA_DTYPE_BF16 && out_dtype != MLA_DTYPE_FP32) return MLA_ERR_BAD_SHAPE;
  if ((reinterpret_cast<uintptr_t>(o_parts) | reinterpret_cast<uintptr_t>(out)) & 15)
    return MLA_ERR_BAD_SHAPE;
  if (rows == 0) return MLA_OK;
  DeviceState *dev;
  if (current_device(&dev) != MLA_OK) return MLA_ERR_DEVICE;
  MergeArgs m;
  m.o_parts = o_parts;
  m.lse_parts = lse_parts;
  m.scale_parts = nullptr;
  m.f16 = 0;
  m.n = n;
  m.rows = rows;
  m.d_v = d_v;
  m.groups = 1;
  m.out = out;
  m.out_fp32 = out_dtype == MLA_DTYPE_FP32 ? 1 : 0;
  m.lse_out = lse_out;
  if (launch_merge(m, static_cast<hipStream_t>(stream)) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

mla_status_t mla_kv_write(const void *rows, const int32_t *slot_mapping, int64_t T, void *kv,
                          int64_t num_slots, const int32_t *positions, int32_t num_shards,
                          int32_t interleave, int32_t shard_id, void *stream) {
  if (T < 0 || num_slots < 1 || num_slots > INT32_MAX) return MLA_ERR_BAD_SHAPE;
  if (num_shards < 1 || num_shards > kMaxShards) return MLA_ERR_BAD_SHAPE;
  if (num_shards > 1 && (interleave < 1 || shard_id < 0 || shard_id >= num_shards)) return MLA_ERR_BAD_SHAPE;
  if (T == 0) return MLA_OK;
  if (!rows || !slot_mapping || !kv || (num_shards > 1 && !positions)) return MLA_ERR_NULL_POINTER;
  if ((reinterpret_cast<uintptr_t>(rows) | reinterpret_cast<uintptr_t>(kv)) & 15) return MLA_ERR_BAD_SHAPE;
  DeviceState *dev;
  if (current_device(&dev) != MLA_OK) return MLA_ERR_DEVICE;
  KvWriteArgs a;
  a.rows = rows;
  a.slots = slot_mapping;
  a.T = T;
  a.kv = kv;
  a.num_slots = num_slots;
  a.positions = positions;
  a.num_shards = num_shards;
  a.interleave = num_shards > 1 ? interleave : 1;
  a.shard_id = num_shards > 1 ? shard_id : 0;
  if (launch_kv_write(a, static_cast<hipStream_t>(stream)) != hipSuccess) return MLA_ERR_LAUNCH;
  return MLA_OK;
}

const char *mla_status_string(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL_POINTER: return "MLA_ERR_NULL_POINTER: a required pointer is NULL";
    case MLA_ERR_BAD_SHAPE: return "MLA_ERR_BAD_SHAPE: a size, stride or alignment is out of range";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: valid arguments this library does not implement";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL: workspace_bytes < mla_workspace_size()";
    case MLA_ERR_LAUNCH: return "MLA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
    case MLA_ERR_DEVICE: return "MLA_ERR_DEVICE: the current HIP device is missing or not a gfx950";
    case MLA_ERR_SCRATCH_LIMIT:
      return "MLA_ERR_SCRATCH_LIMIT: the call needs more scratch than the library's fixed 64 MiB buffer";
  }
  return "unknown mla_status_t";
}

mla_status_t mla_plan_query(const mla_problem_t *problem, int32_t num_shards, int32_t interleave,
                            int32_t shard_id, int32_t top_k, int64_t index_stride_q,
                            int32_t num_cus, mla_plan_t *plan) {
  mla_status_t st = check_problem(problem);
  if (st != MLA_OK) return st;
  if (!plan) return MLA_ERR_NULL_POINTER;
  Plan pl;
  st = make_plan(problem, num_shards, interleave, shard_id, top_k, index_stride_q, num_cus, &pl);
  if (st != MLA_OK) return st;
  plan->q_per_group = pl.q_per_group;
  plan->rows_per_group = pl.rows_per_group;
  plan->units = pl.units;
  plan->splits = pl.splits;
  plan->chunk = pl.chunk;
  plan->stream_len = pl.stream_len;
  plan->grid = pl.grid;
  plan->workspace_bytes = pl.ws_total;
  return MLA_OK;
}

}  // extern "C"
