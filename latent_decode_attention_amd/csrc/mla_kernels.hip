// MLA decode attention kernels for gfx950 (MI355X).
//
// One work-group (4 waves x 64 lanes) owns one (sequence, query group, shard,
// KV partition) unit of up to 64 query rows (query token x head: the heads of
// one token, or whole tokens when heads are few) and streams that unit's latent
// rows through LDS in 64-token tiles.  Every query head dots the same latent row
// (h_kv = 1 for MLA: "RFC: MsModeling 支持 Decode Context Parallel 仿真", §2.1.4
// symbol table), so per tile the work is two dense contractions on the bf16
// matrix cores:
//   scores  S^T[token, row] = K[32 x 576] . Q^T[576 x 32]   wave w: rows 32 (w & 1).., tokens 32 (w >> 1)..
//   output  O^T[col, row]  += V^T[128 x 64] . P^T[64 x 64]  wave w: cols 128 w..128 w + 127
// with V = the first 512 columns of the same LDS rows.  Each wave turns its
// scores into softmax weights P and publishes them in LDS; every wave then
// multiplies all 64 rows' weights against its own quarter of the value
// columns.  Two work-groups cover the 128 heads of a DeepSeek-style query
// token; the KV partitions of a unit and the DCP shards are combined by the
// log-sum-exp merge the DCP page describes (§1.1, §2.1.4.3).
//
// Data movement:
//  * every wave derives the positions, block-table rows (§2.1.4.1, table A) and
//    attended masks of each tile itself: block ids two tiles ahead, positions
//    three tiles ahead, so those loads complete under the math;
//  * tile t+1 is copied HBM -> LDS with direct-to-LDS 16-byte loads spread over
//    tile t's score loops; positions that are padding, out of range or beyond
//    the causal limit are zero-filled in LDS and never read from memory;
//  * an LDS tile holds 64 rows as 9 column groups of 128 bytes (8 chunks of
//    16 bytes): group g of row r lives at g * 8192 + r * 128.  Within a group
//    the chunks of row r are XOR-swizzled by a key of (r / 2) mod 8 chosen so
//    that both the K reads (16 rows, one chunk each, per 16 lanes) and the
//    transposed V reads (4 rows x 4 chunks per 32 lanes) touch every LDS bank
//    exactly once.
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>

#include "mla_internal.h"

// Scratch of the decode entry point that allocates nothing (for callers that
// cannot allocate device memory).  Every device the library runs on holds its
// own copy until the process ends; host code reaches it only through the
// address hipGetSymbolAddress returns for the current device (the name itself
// is a host-side stand-in, not a device address).
static __device__ __align__(256) char scratch[mla::kScratchBytes];

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x16 __attribute__((ext_vector_type(16)));
// Register index of each element of a 16-register MFMA result.
constexpr u32x16 kRegIndex = {0u, 1u, 2u, 3u, 4u, 5u, 6u, 7u, 8u, 9u, 10u, 11u, 12u, 13u, 14u, 15u};
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowBytes = kDqk * 2;            // 1152
constexpr int kChunks = kRowBytes / 16;        // 72
constexpr int kTileBytes = kTile * kRowBytes;  // 73728
constexpr int kQkSteps = kDqk / 16;            // 36 k-steps of the 32x32x16 MFMA
constexpr int kGroups = kChunks / 8;           // 9 column groups of 128 bytes
constexpr int kGroupBytes = kTile * 128;       // 8192
constexpr int kCopySteps = 2 * kGroups;        // direct-load instructions per wave per tile
// int8 cache: a row is 576 bytes; a tile's raw rows fill half a bf16 tile buffer.
constexpr int kRowBytes8 = kDqk;                      // 576
constexpr int kRawTileBytes = kTile * kRowBytes8;     // 36864
constexpr int kCopySteps8 = 16 * kRowBytes8 / 1024;   // 9 direct loads of 1 KiB per wave per tile
static_assert(2 * kRawTileBytes == kTileBytes, "two raw int8 tiles share one bf16 tile buffer");
// Bias of the widened int8 values: byte b is held as b + 128 in [0, 255], an
// integer bf16 represents exactly.
constexpr float kKv8Bias = 128.0f;
// How far (base 2) a score may exceed its row's reference maximum before the
// unit is recomputed with a higher reference: p <= 2^60 keeps sum(p) * |v| far
// inside the fp32 range for any realistic row.
constexpr float kHeadroomLog2 = 60.0f;
// Share of a row's weight from which a token's bf16 rounding in P.V is undone
// at the end (one token's rounding moves O by up to 2^-9 x share x |v - O|) ...
constexpr float kExactShare = 0.25f;
// ... in rows whose output reaches this magnitude in the wave's 128 columns.
// Below it a bf16 output's own rounding (at most 2^-8 there) leaves 0.006 of
// a 1e-2 budget; the two values were chosen on seeded workloads with RoPE-key
// outliers, where rows are dominated by a few tokens.
constexpr float kExactMinOut = 2.0f;
constexpr unsigned kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0), other counters unconstrained

static_assert(kTile == 16 * kWaves, "each wave copies 16 rows of a tile");
static_assert(kWaves == 4, "four waves: four row tiles, or two row tiles x two token halves");

// Source of the bytes copied for tokens that no query row attends, so that a
// tile never holds stale or poisoned rows and the copies need no per-lane branch.
__device__ __attribute__((aligned(256))) const unsigned kZeroRow[kRowBytes / 4] = {};

template <int kRows>
struct __attribute__((aligned(16))) Smem {
  char tile[2][kTileBytes];  // double-buffered latent rows
  // Softmax weights as MFMA B operands: [k-block][row tile][lane].
  bf16x8 p[4][kRows / 32][64];
};
template <>
struct __attribute__((aligned(16))) Smem<64> {
  char tile[2][kTileBytes];
  bf16x8 p[4][2][64];
  float mx[kWaves][32];  // first-tile row maxima exchanged by the two waves of a row tile
  float sig[kTile];      // int8 cache: the current tile's row factors (tiny for unattended tokens)
  float sig_inv[kTile];  // ... and their inverses
};
static_assert(sizeof(Smem<128>) <= 160 * 1024 && sizeof(Smem<64>) <= 160 * 1024, "LDS budget of one work-group");

// ---- Matrix-core helpers.  The 256 output accumulators of a lane fill the
// whole AGPR file, so the MFMAs are written as inline asm with register-class
// constraints (scores in VGPRs, outputs in AGPRs) to keep the allocator from
// shuffling them.  Hazards the compiler cannot see through the asm are covered
// by the fences below (their s_nop counts exceed what the 32x32x16 MFMA needs).
// kGuard: four wait states inside the asm, ahead of the MFMA.  Where the
// register allocator parks operands in AGPRs it copies them back right before
// the asm, too late for any fence in the source; the guard covers those copies.
template <bool kGuard = false>
__device__ __forceinline__ void mfma_vgpr_first(f32x16 &d, bf16x8 a, bf16x8 b) {
  if constexpr (kGuard)
    asm volatile("s_nop 3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
template <bool kGuard = false>
__device__ __forceinline__ void mfma_vgpr(f32x16 &d, bf16x8 a, bf16x8 b) {
  if constexpr (kGuard)
    asm volatile("s_nop 3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
template <bool kGuard = false>
__device__ __forceinline__ void mfma_agpr(f32x16 &d, bf16x8 a, bf16x8 b) {
  if constexpr (kGuard)
    asm volatile("s_nop 3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// Zero a 16-register accumulator tile without touching VGPRs: 0 x 0 + 0.
__device__ __forceinline__ void acc_zero(f32x16 &d, bf16x8 z) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(d) : "v"(z));
}
// MFMA result -> VALU reads.
__device__ __forceinline__ void mfma_result_fence(f32x16 &d) {
  asm volatile("s_nop 15\n\ts_nop 3" : "+v"(d));
}
// VALU-written VGPRs -> MFMA operand reads.
__device__ __forceinline__ void operand_fence(bf16x8 &a) { asm volatile("s_nop 3" : "+v"(a)); }
template <int kTiles>
__device__ __forceinline__ void acc_result_fence(f32x16 *acc) {
  asm volatile("s_nop 15\n\ts_nop 3" ::: "memory");
#pragma unroll
  for (int i = 0; i < kTiles; ++i) asm volatile("" : "+a"(acc[i]));
}

// Work-group barrier that orders LDS accesses only.  __syncthreads() also
// waits for this wave's outstanding global stores (a full memory round trip),
// which the epilogue's LDS exchange does not need.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Chunk key of tile row r: 0, 4, 1, 5, 2, 6, 3, 7 for (r / 2) mod 8.  Even rows
// and odd rows sit in opposite halves of the 64 banks, so a K read (rows
// r0..r0+15 at one logical chunk) is conflict-free when the 8 even rows, and the
// 8 odd rows, have distinct keys; a transposed V read (rows r0..r0+3, chunks
// 4 j .. 4 j + 3) when rows r and r + 2 differ in key bit 2.  The key repeats
// every 16 rows, so sub-block and k-block offsets keep it.
__device__ __forceinline__ int chunk_key(int row) {
  const int m = (row >> 1) & 7;
  return ((m & 1) << 2) | (m >> 1);
}

__device__ __forceinline__ int shard_len(int S, int N, int I, int r) {
  if (S <= 0) return 0;
  const int full = S / I, rem = S % I;
  const int groups = full > r ? (full - 1 - r) / N + 1 : 0;
  return groups * I + ((full % N) == r ? rem : 0);
}

// How a unit's token stream maps to positions: every position, the positions
// of one DCP shard, or a top-k index list.
enum StreamMode { kDenseStream = 0, kShardStream = 1, kSparseStream = 2 };

struct Unit {
  int b, q0, shard, split;
  int unit;       // (sequence, query group, shard) index: work-group id / splits
  int h0, rows;   // first head and number of query rows of the group
  int64_t row0;   // flattened (query token, head) row of the group's row 0
  int S, i0, i1;
  int64_t idx_base;
  const int32_t *list;  // sparse: the list the stream indexes (idx_base on)
  const int32_t *bt;    // this sequence's block-table row
};

// Values the compiler cannot prove wave-uniform (loads from memory the kernel
// might also write, 64-bit products) are moved to scalar registers explicitly.
// Pointers stay kernel-argument base + uniform offset, so the compiler still
// knows they address global memory.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform(int64_t v) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Sparse under DCP: the entries of the unit's list that belong to `shard`
// (valid positions p, 0 <= p < S, with floor(p / interleave) mod num_shards =
// shard), in list order ("RFC: MsModeling 支持 Decode Context Parallel 仿真",
// §2.1.4.1, interleaved placement).  Returns their number L; those of ranks
// [i0, i1) (i1 = L for the unit's last partition, else min(L, i0 + chunk)),
// this partition's share, are stored at dst[rank].  Every thread of the
// work-group takes part: wave w scans a quarter of the list, counting, then
// again placing its entries after the earlier quarters' counts.  `cnt` is LDS
// scratch of kWaves ints.
constexpr int kSelectBatch = 8;  // 64-entry rounds per batch of loads (a whole 2048-entry list)
__device__ __forceinline__ int select_shard_entries(const DecodeArgs &a, const int32_t *src, int S, unsigned shard,
                                                    int i0, int chunk, bool last, int32_t *dst, int *cnt) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int quarter = (a.top_k + kWaves * 64 - 1) / (kWaves * 64) * 64;
  const int lo = wave * quarter, hi = min(a.top_k, lo + quarter);
  auto owned = [&](int i, int p) {
    const unsigned run = fastdiv((unsigned)p, a.by_interleave);
    const unsigned owner = run - fastdiv(run, a.by_shards) * (unsigned)a.num_shards;
    return i < hi && p >= 0 && p < S && owner == shard;
  };
  // Each batch issues all its loads (clamped addresses) before the first use.
  auto scan = [&](auto visit) {
    for (int b0 = lo; b0 < hi; b0 += 64 * kSelectBatch) {
      int v[kSelectBatch];
#pragma unroll
      for (int j = 0; j < kSelectBatch; ++j) v[j] = src[min(b0 + 64 * j + lane, a.top_k - 1)];
#pragma unroll
      for (int j = 0; j < kSelectBatch; ++j) visit(owned(b0 + 64 * j + lane, v[j]), v[j]);
    }
  };
  int count = 0;
  scan([&](bool m, int) { count += __popcll(__ballot(m)); });
  if (lane == 0) cnt[wave] = count;
  __syncthreads();
  int rank = 0, L = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int c = cnt[w];
    rank += w < wave ? c : 0;
    L += c;
  }
  const int i1 = last ? L : min(L, i0 + chunk);
  scan([&](bool m, int p) {
    const unsigned long long bm = __ballot(m);
    const int r = rank + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bm >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((unsigned)bm, 0u));
    if (m && r >= i0 && r < i1) dst[r] = p;
    rank += __popcll(bm);
  });
  // The stored entries are read back by other waves of the work-group.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  return L;
}

template <int kMode>
__device__ __forceinline__ Unit decode_unit(const DecodeArgs &a, int *lds_scratch) {
  const uint32_t grid = gridDim.x;  // < 2^31 (the plan checks)
  uint32_t id = blockIdx.x;
  // Work-groups are dealt round-robin to the 8 XCDs; renumber so that the
  // partitions of one unit (which share the unit's query rows) sit on one XCD.
  if ((grid & 7) == 0) id = (id & 7) * (grid >> 3) + (id >> 3);
  // 32-bit unsigned arithmetic: the 64-bit divisions this replaced were a long
  // branchy sequence in front of the first loads.
  Unit u;
  const uint32_t splits = a.splits, q_groups = a.q_groups, shard_units = a.shard_units, head_chunks = a.head_chunks;
  u.split = (int)(id % splits);
  id /= splits;
  u.unit = (int)id;
  const uint32_t qg = id % q_groups;
  id /= q_groups;
  const int su = (int)(id % shard_units);
  u.b = (int)(id / shard_units);
  u.q0 = (int)(qg / head_chunks) * a.q_per_group;
  u.h0 = (int)(qg % head_chunks) * a.rows_per_group;
  u.rows = min(a.rows_per_group, a.q_per_group * a.h_q - u.h0);
  u.row0 = uniform(((int64_t)u.b * a.Q + u.q0) * a.h_q + u.h0);
  u.shard = a.shard_base + su;
  if constexpr (kMode == kSparseStream) {
    // Only the causal checks, after the first index and block loads, use the
    // length: read it with a vector load and leave it in a register, so that
    // no wait on scalar loads in front of those loads covers it.
    int bl = u.b;
    asm volatile("" : "+v"(bl));
    u.S = a.seq_lens[bl];
  } else {
    u.S = uniform(a.seq_lens[u.b]);
  }
  int L;
  u.idx_base = 0;
  bool rest = false;  // the last partition also takes what the plan did not foresee
  if constexpr (kMode == kSparseStream) {
    const int64_t src = uniform((int64_t)u.b * a.idx_stride_b + (int64_t)u.q0 * a.idx_stride_q);
    if (a.own_lists) {
      // This shard's entries of the list; their number is known only on the
      // device.  The plan cuts partitions for an even share of the entries
      // per shard, and the last partition takes whatever is beyond.
      rest = u.split == a.splits - 1;
      u.idx_base = uniform((int64_t)u.unit * a.top_k);
      u.list = a.own_lists;
      L = uniform(select_shard_entries(a, a.indices + src, u.S, (unsigned)u.shard, u.split * a.chunk, a.chunk, rest,
                                       a.own_lists + u.idx_base, lds_scratch));
    } else {
      L = a.top_k;
      u.idx_base = src;
      u.list = a.indices;
    }
  } else if constexpr (kMode == kShardStream) {
    L = shard_len(u.S, a.num_shards, a.interleave, u.shard);
  } else {
    L = u.S > 0 ? u.S : 0;
  }
  u.i0 = uniform(u.split * a.chunk);
  u.i1 = uniform(rest ? L : min(L, u.i0 + a.chunk));
  u.bt = a.block_table + uniform((int64_t)u.b * a.max_blocks);
  return u;
}

// ---- Per-tile token metadata, one token per lane.  The raw loads use clamped
// (always in-bounds) addresses and are examined only after the tile's math, so
// no wait on them lands in front of the math (a wait there would also drain
// the in-flight copy of the next tile, which shares the vector-memory counter).

// Stream index i -> logical position (dense: the position itself or the i-th
// position the shard owns; sparse: the raw list entry, validated later).
template <int kMode>
__device__ __forceinline__ int raw_position(const DecodeArgs &a, const Unit &u, int i) {
  if constexpr (kMode == kSparseStream) return u.list[u.idx_base + min(i, u.i1 - 1)];
  if constexpr (kMode == kShardStream)
    return ((i / a.interleave) * a.num_shards + u.shard) * a.interleave + (i % a.interleave);
  return i;
}
__device__ __forceinline__ int raw_block(const DecodeArgs &a, const Unit &u, int p) {
  const int slot = min(max(p, 0) >> a.bs_shift, a.max_blocks - 1);
  return u.bt[slot];
}
// Physical cache row of a token, or -1 when no query row of this group attends
// it.  (Under DCP, streams hold only positions of their own shard: dense
// streams by construction, sparse ones by select_shard_entries.)
__device__ __forceinline__ int token_row(const DecodeArgs &a, const Unit &u, int i, int p, int blk) {
  const int last = u.S - a.Q + u.q0 + a.q_per_group - 1;
  const bool ok = i < u.i1 && p >= 0 && p <= last && (p >> a.bs_shift) < a.max_blocks && blk >= 0 &&
                  blk < a.num_blocks;
  return ok ? blk * a.block_size + (p & (a.block_size - 1)) : -1;
}

// Attended-token bitmask of one tile for each query token of the group.
struct TileMask {
  unsigned long long m[kMaxQPerGroup];
  bool full;  // every token attended by every query token of the group
};
__device__ __forceinline__ TileMask tile_mask(const DecodeArgs &a, const Unit &u, int p, int row) {
  TileMask t;
  unsigned long long all = ~0ull;
#pragma unroll
  for (int qq = 0; qq < kMaxQPerGroup; ++qq) {
    // Query tokens past the group's own attend nothing: a limit of -1,
    // chosen on the scalar unit rather than by branching around the ballot.
    const int lim = qq < a.q_per_group ? u.S - a.Q + u.q0 + qq : -1;
    t.m[qq] = __ballot(row >= 0 && p <= lim);
    all &= qq < a.q_per_group ? t.m[qq] : ~0ull;
  }
  t.full = all == ~0ull;
  return t;
}

// ---- Direct global -> LDS copies.  One instruction moves 16 bytes per lane:
// lane l's bytes land at LDS address M0 + 16 l.  Issued as inline asm so that
// the compiler's memory model does not order it against the other buffer's LDS
// reads (it would otherwise drain vmcnt before every LDS access); completion is
// awaited explicitly with s_waitcnt vmcnt(0) before the barrier that publishes
// the tile.  m0 is reserved for the compiler, which uses it for nothing else in
// these kernels; the clobber records that the copy rewrites it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// M0 = lds_base + lds_off (an immediate once the copy loop is unrolled), one
// wait state for the M0 write to reach the direct load, then the load.
// The source offset is the instruction's immediate (a constant up to 1 KiB here,
// within its signed 13-bit range), so a copy needs no address arithmetic.  The
// immediate is added to the LDS address as well as to the global one, so M0 is
// set that much lower.
template <int kSrcOff, int kLdsOff>
__device__ __forceinline__ void dma16(const char *src, unsigned lds_base) {
  static_assert(kSrcOff >= 0 && kSrcOff < 4096, "immediate offset range");
  static_assert(kLdsOff >= kSrcOff, "M0 offset stays non-negative");
  asm volatile("s_add_u32 m0, %0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:%3"
               :
               : "s"(lds_base), "v"(src), "i"(kLdsOff - kSrcOff), "i"(kSrcOff)
               : "m0");
}
#pragma clang diagnostic pop

// Copy of one tile: wave w copies rows 16w..16w+15; step j moves 8 rows x 128
// bytes of column group j % 9 of the 8-row block j / 9, lane l taking row
// 16w + 8 (j / 9) + l / 8 and stored position l % 8 of it.  Rows nobody
// attends (row index -1) are copied from the zero row.
struct TileCopy {
  const char *src[2];  // this lane's 16 source bytes in each 8-row block, group 0
  unsigned lds[2];     // wave-uniform LDS address of each 8-row block, group 0
};

// The cache rows of the two tokens lane l copies: tokens 16 w + 8 k + l / 8 of
// the tile, fetched from the lanes that derived them (lane = token).
struct CopyRows {
  int row[2];
};
__device__ __forceinline__ CopyRows copy_rows(int tile_row, int wave, int lane) {
  CopyRows r;
#pragma unroll
  for (int k = 0; k < 2; ++k) r.row[k] = __shfl(tile_row, 16 * wave + 8 * k + (lane >> 3));
  return r;
}
__device__ __forceinline__ TileCopy copy_from_rows(char *tile_buf, const DecodeArgs &a, int wave, int lane,
                                                   const CopyRows &r) {
  TileCopy c;
  // Cheap per-lane constants, recomputed on every call (opaque copy of the lane)
  // rather than hoisted out of the tile loop and held in registers.
  int l = lane;
  asm volatile("" : "+v"(l));
  const int sub = l >> 3;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int chunk = ((l & 7) ^ chunk_key(8 * k + sub)) * 16;
    const int row = r.row[k];
    // Both candidates are formed and one is selected, so no branch or exec-mask
    // change is needed (unattended tokens read the zero row).
    const char *row_src = reinterpret_cast<const char *>(a.kv) + (int64_t)max(row, 0) * kRowBytes;
    c.src[k] = (row < 0 ? reinterpret_cast<const char *>(kZeroRow) : row_src) + chunk;
    const unsigned blk = (unsigned)(uintptr_t)(tile_buf + (16 * wave + 8 * k) * 128);
    c.lds[k] = __builtin_amdgcn_readfirstlane(blk);
  }
  return c;
}
__device__ __forceinline__ TileCopy prepare_copy(char *tile_buf, const DecodeArgs &a, int wave, int lane,
                                                 int tile_row) {
  return copy_from_rows(tile_buf, a, wave, lane, copy_rows(tile_row, wave, lane));
}

template <int kJ>
__device__ __forceinline__ void copy_step(const TileCopy &c) {
  constexpr int k = kJ / kGroups, g = kJ % kGroups;
  dma16<g * 128, g * kGroupBytes>(c.src[k], c.lds[k]);
}
template <int... kJ>
__device__ __forceinline__ void copy_steps(const TileCopy &c, std::integer_sequence<int, kJ...>) {
  (copy_step<kJ>(c), ...);
}
__device__ __forceinline__ void copy_all(const TileCopy &c) {
  copy_steps(c, std::make_integer_sequence<int, kCopySteps>());
}
// Copy step j where j is a constant once the tile loop is unrolled (the
// comparisons then fold to the one call).
template <int... kJ>
__device__ __forceinline__ void copy_step_at(const TileCopy &c, int j, std::integer_sequence<int, kJ...>) {
  ((j == kJ ? copy_step<kJ>(c) : void()), ...);
}

// Copy of one int8 tile into a raw buffer: wave w copies rows 16w..16w+15 into
// its 9 KiB slice; step j moves bytes 64 j .. 64 j + 63 of each of the 16 rows,
// lane l taking row 16 w + l / 4 and its bytes 64 j + 16 (l % 4), which land at
// 1024 j + 16 l.  Raw 16-byte chunk C of wave row rho therefore sits at
// 1024 (C / 4) + 64 rho + 16 (C % 4) of the slice.
struct TileCopy8 {
  const char *src;  // this lane's row + 16 (l % 4); the step's 64 j is the immediate
  unsigned lds;     // wave-uniform LDS address of the wave's slice
};
__device__ __forceinline__ TileCopy8 prepare_copy8(char *raw_buf, const DecodeArgs &a, int wave, int lane,
                                                   int tile_row) {
  int l = lane;
  asm volatile("" : "+v"(l));
  const int row = __shfl(tile_row, 16 * wave + (l >> 2));
  const char *row_src = reinterpret_cast<const char *>(a.kv) + (int64_t)max(row, 0) * kRowBytes8;
  TileCopy8 c;
  c.src = (row < 0 ? reinterpret_cast<const char *>(kZeroRow) : row_src) + 16 * (l & 3);
  c.lds = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(raw_buf + wave * 16 * kRowBytes8));
  return c;
}
template <int kJ>
__device__ __forceinline__ void copy_step8(const TileCopy8 &c) {
  dma16<64 * kJ, 1024 * kJ>(c.src, c.lds);
}
template <int... kJ>
__device__ __forceinline__ void copy_all8(const TileCopy8 &c, std::integer_sequence<int, kJ...>) {
  (copy_step8<kJ>(c), ...);
}
template <int... kJ>
__device__ __forceinline__ void copy_step8_at(const TileCopy8 &c, int j, std::integer_sequence<int, kJ...>) {
  ((j == kJ ? copy_step8<kJ>(c) : void()), ...);
}

// acc + lo(w) + hi(w) for a packed bf16 pair w (v_dot2c_f32_bf16 with (1, 1)).
// Written as asm: the compiler's own lowering of the dot2 builtin misplaced its
// operands in this kernel.
__device__ __forceinline__ float sum_bf16_pair(float acc, unsigned w, unsigned ones) {
  asm("v_dot2c_f32_bf16 %0, %1, %2" : "+v"(acc) : "v"(w), "v"(ones));
  return acc;
}

// Two floats to packed bf16 (round to nearest even, v_cvt_pk_bf16_f32).  Vectors
// of bf16 are only ever assembled from whole 32-bit words: inserting single
// __bf16 elements into a vector miscompiles with this toolchain.
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Two floats to packed fp16 (round to nearest even).
__device__ __forceinline__ unsigned pack_f16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, f16x2));
}

__device__ __forceinline__ float half_bits_to_float(unsigned bits) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)bits);
}

// Element types of an output or partial buffer.
enum OutKind { kOutBf16 = 0, kOutFp32 = 1, kOutFp16 = 2 };

__device__ __forceinline__ void store_out(void *out, int kind, int64_t elem, f32x4 v) {
  if (kind == kOutFp32) {
    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + elem) = v;
  } else if (kind == kOutBf16) {
    const u32x2 h = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    *reinterpret_cast<u32x2 *>(reinterpret_cast<__bf16 *>(out) + elem) = h;
  } else {
    const u32x2 h = {pack_f16(v[0], v[1]), pack_f16(v[2], v[3])};
    *reinterpret_cast<u32x2 *>(reinterpret_cast<_Float16 *>(out) + elem) = h;
  }
}

// Widen the wave's 16 rows of a raw int8 tile into the bf16 tile layout.  Byte
// b becomes b + 128 (XOR 0x80 reads the signed byte as that unsigned value),
// exact in bf16; the kernel takes the bias back out of the scores and outputs.
// Pass (h, g) covers 8 rows x the 8 chunks of column group g: lane l reads 8 raw
// bytes (512 contiguous bytes per wave) and writes one 16-byte chunk (each 16
// lanes write two whole 128-byte rows: every bank once).  The 9 reads of a half
// are issued together, so their latency is paid twice per tile, not 18 times.
__device__ __forceinline__ void widen_tile8(const char *raw_buf, char *tile_buf, int wave, int lane) {
  const char LDS_AS *src = (const char LDS_AS *)(raw_buf + wave * 16 * kRowBytes8 + 8 * lane);
  const int c = lane & 7;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rr = 8 * h + (lane >> 3);  // row within the wave's 16; its key is that of 16 wave + rr
    char LDS_AS *dst = (char LDS_AS *)(tile_buf + (16 * wave + rr) * 128 + 16 * (c ^ chunk_key(rr)));
    unsigned rl[kGroups], rh[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const u32x2 w = *(const u32x2 LDS_AS *)(src + g * 1024 + h * 512);
      rl[g] = w[0];
      rh[g] = w[1];
    }
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const unsigned lo = rl[g] ^ 0x80808080u, hi = rh[g] ^ 0x80808080u;
      const u32x4 o = {pack_bf16((float)(lo & 255u), (float)((lo >> 8) & 255u)),
                       pack_bf16((float)((lo >> 16) & 255u), (float)(lo >> 24)),
                       pack_bf16((float)(hi & 255u), (float)((hi >> 8) & 255u)),
                       pack_bf16((float)((hi >> 16) & 255u), (float)(hi >> 24))};
      *(u32x4 LDS_AS *)(dst + g * kGroupBytes) = o;
    }
  }
}

// Power-of-two scale for storing values of magnitude up to `vmax` as fp16: the
// largest lands in [2^14, 2^15), so every value keeps fp16's 11-bit precision
// down to 2^-28 of the maximum.  Returns the scale; *inv gets its exact inverse.
__device__ __forceinline__ float fp16_scale(float vmax, float *inv) {
  int e = (int)((__builtin_bit_cast(unsigned, vmax) >> 23) & 255u) - 127;
  e = max(-110, min(e, 127));
  *inv = __builtin_bit_cast(float, (unsigned)(e - 14 + 127) << 23);
  return __builtin_bit_cast(float, (unsigned)(14 - e + 127) << 23);
}

// kRows = 128: wave w scores rows 32 w.. against both 32-token halves of each
// tile in turn (two sub-blocks) and owns those rows' softmax state outright.
// kRows = 64: wave w scores row tile w & 1 against token half w >> 1 only, so
// the two waves of a row tile (w, w ^ 2) agree on the rows' reference maximum
// at the first tile and combine their sums at the end.
//
// kKv8 (int8 cache, 64 rows only): the raw rows of tiles t and t+1 are
// double-buffered in the first tile buffer; at the top of tile t each wave
// widens its own 16 rows into the second buffer, which the scores and P.V read
// as with a bf16 cache.  Scores are sigma_p (s'_p - 128 sum(q)) with s' the
// product against the biased values; the weights fed to P.V carry sigma_p, and
// the outputs drop 128 x (sum of those weights) before normalising by the sum
// of the weights over their factors.
template <int kMode, int kRows, bool kKv8 = false>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(const DecodeArgs a) {
  static_assert(!kKv8 || kRows == 64, "int8 tiles leave LDS for 64-row work-groups only");
  constexpr int kRowTiles = kRows / 32;
  constexpr int kAccTiles = 4 * kRowTiles;  // row tiles x 4 column tiles of 32 x 32
  constexpr int kSubBlocks = kRows / 64;    // 32-token score blocks per wave per tile
  constexpr int kPvSteps = 16;               // (k-block, column tile) steps of P.V
  constexpr int kCopyFirst = 3;              // first step that copies (after its addresses are formed)
  // K operand reads in flight ahead of the MFMA that uses them: deep enough for
  // the LDS latency while the copies land (64-row bf16 kernels); the 128-row
  // and int8 kernels have no registers to spare for more than three.
  constexpr int kKAhead = kRows == 64 && !kKv8 ? 5 : 3;
  constexpr int kSteps = kKv8 ? kCopySteps8 : kCopySteps;  // copy instructions per wave per tile
  constexpr int kCopyEvery = (kSubBlocks * kQkSteps + kPvSteps - kCopyFirst) / kSteps;
  static_assert(kCopyFirst + kCopyEvery * (kSteps - 1) < kSubBlocks * kQkSteps + kPvSteps,
                "the copy of the next tile is issued within the tile");
  __shared__ Smem<kRows> sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, half = lane >> 5;
  const int rh = kRows == 128 ? wave : (wave & 1);  // the wave's row tile for the scores
  const int th = kRows == 128 ? 0 : (wave >> 1);    // its token half (64 rows)

  const Unit u = decode_unit<kMode>(a, reinterpret_cast<int *>(sm.tile[1]));
  const int ntiles = u.i1 > u.i0 ? (u.i1 - u.i0 + kTile - 1) / kTile : 0;

  // Output destination: final tensor or this partition's slot of the partials.
  const int64_t su = u.shard - a.shard_base;
  void *obase;
  float *lbase;
  float *sbase = nullptr;  // fp16 partials: inverse scale per (row, column quarter)
  int okind;
  if (a.splits > 1) {
    const int64_t g = uniform((su * a.splits + u.split) * a.rows_total);
    if (a.part_f16) {
      okind = kOutFp16;
      obase = reinterpret_cast<_Float16 *>(a.part_o) + g * kDv;
      sbase = a.part_scale + g * kWaves;
    } else {
      okind = kOutFp32;
      obase = reinterpret_cast<float *>(a.part_o) + g * kDv;
    }
    lbase = a.part_lse + g;
  } else {
    const int64_t g = uniform(su * a.rows_total);
    okind = a.out_fp32 ? kOutFp32 : kOutBf16;
    obase = a.out_fp32 ? (void *)(reinterpret_cast<float *>(a.out) + g * kDv)
                       : (void *)(reinterpret_cast<__bf16 *>(a.out) + g * kDv);
    lbase = a.lse + g;
  }
  // Global row (query token x head, flattened) of the group's row r.
  auto out_row = [&](int r) -> int64_t { return u.row0 + r; };

  const int row_local = 32 * rh + n;
  const bool row_ok = row_local < u.rows;

  if (ntiles == 0) {
    // Nothing attended: O = 0, lse = -inf (written by the token-half-0 waves).
    if (th == 0 && row_ok) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const int64_t gr = out_row(row_local);
      for (int c = half * 4; c < kDv; c += 8) store_out(obase, okind, gr * kDv + c, z);
      if (half == 0) {
        lbase[gr] = -INFINITY;
        if (okind == kOutFp16)
          for (int w = 0; w < kWaves; ++w) sbase[gr * kWaves + w] = 1.f;
      }
    }
    return;
  }
  // Query token of the row within the group (heads of one token are contiguous).
  const int q_local = row_ok ? (u.h0 + row_local) / a.h_q : 0;

  // ---- Start of a pass: the memory chain positions -> block ids -> rows ->
  // copy of tile 0, with the positions of tiles 0..2 and the block ids of
  // tiles 0 and 1 each fetched in one round trip.  Leaves the masks of tile 0
  // and the raw lookups of tiles 1 and 2 for the tile loop.  (The opaque lane
  // copy keeps this per-pass work from being hoisted and held in registers.)
  // `between` runs after the positions and `after_blocks` after the block ids
  // are issued: the first pass loads the query rows there, so each wait of
  // the chain leaves the query loads issued after it in flight.
  // `before_copy` runs once the rows are known, before the copy of tile 0 is
  // issued (64-row groups stage their query halves in LDS there, so that the
  // exchange of the halves overlaps the copy in flight instead of following
  // it; any wait on a load placed after the copies would drain them too).
  TileMask mask_cur;
  int pn1, bn1, pn2;
  int row_cur = -1;  // 64-row groups: cache row of this lane's token (lane = token) in the current tile
  // int8 cache: the row factor each lane (= token) loaded for the current tile,
  // and whether its token is attended at all (else the factor is taken as 0).
  float sig_raw = 0.f;
  bool sig_ok = false;
  auto start_pass = [&](auto between, auto after_blocks, auto before_copy) {
    int plane = lane;
    asm volatile("" : "+v"(plane));
    const int p0 = raw_position<kMode>(a, u, u.i0 + plane);
    pn1 = raw_position<kMode>(a, u, u.i0 + kTile + plane);
    pn2 = raw_position<kMode>(a, u, u.i0 + 2 * kTile + plane);
    __builtin_amdgcn_sched_barrier(0);  // keep the load order: each wait below
    between();                          // then leaves the later loads in flight
    __builtin_amdgcn_sched_barrier(0);
    const int b0 = raw_block(a, u, p0);
    bn1 = raw_block(a, u, pn1);
    __builtin_amdgcn_sched_barrier(0);
    after_blocks();
    __builtin_amdgcn_sched_barrier(0);
    const int row0 = token_row(a, u, u.i0 + plane, p0, b0);
    if constexpr (kRows == 64) row_cur = row0;
    before_copy();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kKv8) {
      copy_all8(prepare_copy8(sm.tile[0], a, wave, lane, row0), std::make_integer_sequence<int, kCopySteps8>());
      sig_raw = a.kv_scale[max(row0, 0)];
      sig_ok = row0 >= 0;
    } else {
      copy_all(prepare_copy(sm.tile[0], a, wave, lane, row0));
    }
    mask_cur = tile_mask(a, u, p0, row0);
  };

  // Query rows in registers: lane (n, half) holds q[row][16 st + 8 half + 0..7], the
  // B operand of the 32x32x16 MFMA for k-step st, loaded in two halves inside
  // the first pass's lookup chain; the first tile's wait covers them.  Rows
  // past the group's end load the group's first row instead (no branch around
  // the loads); their outputs are never stored.
  bf16x8 qr[kQkSteps];
  const bf16x8 *qp = reinterpret_cast<const bf16x8 *>(a.q + out_row(row_ok ? row_local : 0) * kDqk);
  if constexpr (kRows == 128) {
    start_pass(
        [&]() {
#pragma unroll
          for (int st = 0; st < kQkSteps / 2; ++st) qr[st] = qp[2 * st + half];
        },
        [&]() {
#pragma unroll
          for (int st = kQkSteps / 2; st < kQkSteps; ++st) qr[st] = qp[2 * st + half];
        },
        []() {});
  } else {
    // The two waves of a row tile hold the same query rows: each loads half of
    // the k-steps (token half th: k-steps 18 th..18 th+17, chosen through the
    // address so register indices stay compile-time) and the halves meet in
    // the idle second tile buffer, [row tile][k-step][lane] x 16 bytes =
    // exactly one tile buffer.  Halves the query loads at the start of the
    // kernel, which share the vector memory pipeline with its lookup chain.
    constexpr int kHalf = kQkSteps / 2;
    bf16x8 tq[kHalf];
    const bf16x8 *qsrc = qp + 2 * kHalf * th;
    bf16x8 *q_sh = reinterpret_cast<bf16x8 *>(sm.tile[1]) + rh * kQkSteps * 64 + lane;
    start_pass(
        [&]() {
#pragma unroll
          for (int j = 0; j < kHalf / 2; ++j) tq[j] = qsrc[2 * j + half];
        },
        [&]() {
#pragma unroll
          for (int j = kHalf / 2; j < kHalf; ++j) tq[j] = qsrc[2 * j + half];
        },
        [&]() {
          // The halves (issued after the block ids, landing about with them)
          // go to LDS before tile 0 is copied; the compiler's waits for them
          // then cover no direct copy.
#pragma unroll
          for (int j = 0; j < kHalf; ++j) q_sh[(kHalf * th + j) * 64] = tq[j];
        });
    lds_barrier();  // every wave's half is in LDS (tile 0 may still be in flight)
#pragma unroll
    for (int st = 0; st < kQkSteps; ++st) qr[st] = q_sh[st * 64];
    // (The first tile's top barrier orders these reads before any copy into
    // the buffer.)
  }

  // Per-lane LDS byte offsets within a tile.  K step st reads logical chunk
  // 2 st + half of row 32 th + n: with the row's XOR key that is column group
  // st / 4 (an immediate) plus the per-lane base with its chunk bits flipped by
  // 2 (st % 4).  V reads of k-block kb and column tile ct: rows
  // 16 kb + 4 half + (lane & 15) / 4 (second read: + 8), columns
  // 128 wave + 32 ct + 16 ((lane >> 4) & 1) + 4 (lane & 3): column group
  // 2 wave + ct / 2 plus the per-lane base (one per read, the two rows having
  // different keys) with chunk bit 2 flipped for odd ct.
  const int k_base = th * 32 * 128 + n * 128 + (((half ^ chunk_key(n)) & 7) << 4);
  const int v_row = 4 * half + ((lane & 15) >> 2);
  const int v_lc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int v_base = 2 * wave * kGroupBytes + v_row * 128 + (((v_lc ^ chunk_key(v_row)) & 7) << 4) + 8 * (lane & 1);
  const int v_base8 =
      2 * wave * kGroupBytes + (v_row + 8) * 128 + (((v_lc ^ chunk_key(v_row + 8)) & 7) << 4) + 8 * (lane & 1);
  const bf16x8 zero8 = {};
  unsigned ones2 = 0x3F803F80u;  // (1.0, 1.0) in bf16, kept in a register
  asm volatile("" : "+v"(ones2));
  // int8 cache: 128 x (sum of the row's query elements), the part of each score
  // that the bias of the widened values adds.
  float q_bias = 0.f;
  if constexpr (kKv8) {
#pragma unroll
    for (int st = 0; st < kQkSteps; ++st) {
      const u32x4 w = __builtin_bit_cast(u32x4, qr[st]);
#pragma unroll
      for (int e = 0; e < 4; ++e) q_bias = sum_bf16_pair(q_bias, w[e], ones2);
    }
    q_bias = (q_bias + __shfl_xor(q_bias, 32)) * kKv8Bias;
  }

  // Softmax bookkeeping for this wave's 32 rows, base-2 units.  m_ref is the
  // row's reference maximum, raised only by a recompute pass (to the largest
  // score seen).  128 rows: set from the first sub-block in which the row
  // attends anything.  64 rows: common to the row's two waves, the larger of
  // their first-tile maxima; a row first attending later forces a recompute.
  // p = 2^(x - m_ref) may exceed 1 by up to 2^kHeadroomLog2, which fp32
  // accumulators and bf16 operands carry without loss, so the accumulators are
  // never rescaled; a score beyond that headroom sends the unit through a
  // recompute pass.
  float m_ref = -INFINITY;
  float l_run = 0.f;         // this lane's share of sum(p), for lse
  float l_rnd = 0.f;         // the same sum over p as rounded to bf16, for O
  float l_cvx = 0.f;         // int8 cache: sum of the rounded weights over their row factors, for O
  f32x16 acc[kAccTiles];     // acc[4 rt + ct]: rows 32 rt.., columns 128 wave + 32 ct..
  bool first_pass = true;
  // The lane's largest score of the pass and its token (64-row groups: the
  // token's cache row; 128-row groups: its index in the unit's stream).
  // Every score carries its register index in its 4 lowest mantissa bits (a
  // change of at most 2^-19 of the score), so a maximum also names its token:
  // the finalize step restores that token's exact weight (see there).
  float best_x = -INFINITY;
  int best_row = -1;

  for (;;) {
    bf16x8 z = zero8;
    operand_fence(z);  // the zero operand may have just been written by a VALU move
#pragma unroll
    for (int i = 0; i < kAccTiles; ++i) acc_zero(acc[i], z);
    l_run = 0.f;
    l_rnd = 0.f;
    l_cvx = 0.f;
    best_x = -INFINITY;
    best_row = -1;
    bool overflow = false;

    for (int t = 0; t < ntiles; ++t) {
      const int cur = t & 1;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's copies of tile t have landed
      __syncthreads();                       // ... every wave's; tile t-1's P and V are consumed
      if constexpr (kKv8) {
        if (wave == 0) {
          // A zero factor (and an unattended token) is replaced by 2^-100 so
          // that its inverse is finite: the token's weight still counts in the
          // normaliser while its values contribute nothing measurable.
          const float f = sig_ok && sig_raw != 0.f ? sig_raw : 0x1p-100f;
          sm.sig[lane] = f;
          sm.sig_inv[lane] = 1.f / f;
        }
        widen_tile8(sm.tile[0] + cur * kRawTileBytes, sm.tile[1], wave, lane);
        lds_barrier();  // the widened tile and its factors are in LDS
      }
      // Tile t+1's rows and masks (from lookups that landed with the wait
      // above), its copy addresses, and the raw lookups two and three tiles
      // ahead are worked out during the first score steps, in the MFMAs'
      // shadow; the lookups are examined only at the next tile's top (after its
      // wait), so no wait on them falls inside this tile.  The copy of tile t+1
      // then issues one instruction every kCopyEvery steps from step
      // kCopyFirst on (its addresses come first), through the scores.  After the
      // last tile every row is -1 and the copy moves zero rows into the idle
      // buffer (drained after the loop), which avoids a branch per copy.
      int row1 = -1, bn2 = 0, pn3 = 0;
      float sig1_raw = 0.f;
      bool sig1_ok = false;
      TileMask mask1;
      CopyRows crow;
      TileCopy next_copy;
      TileCopy8 next_copy8;
      auto tile_step_work = [&](int step) {
        if (step == 0) {
          row1 = token_row(a, u, u.i0 + (t + 1) * kTile + lane, pn1, bn1);
          if constexpr (kKv8) {
            sig1_raw = a.kv_scale[max(row1, 0)];
            sig1_ok = row1 >= 0;
          } else {
            crow = copy_rows(row1, wave, lane);
          }
        }
        if (step == 2) {
          if constexpr (kKv8)
            next_copy8 = prepare_copy8(sm.tile[0] + (cur ^ 1) * kRawTileBytes, a, wave, lane, row1);
          else
            next_copy = copy_from_rows(sm.tile[cur ^ 1], a, wave, lane, crow);
        }
        if (step == 4) {
          bn2 = raw_block(a, u, pn2);
          pn3 = raw_position<kMode>(a, u, u.i0 + (t + 3) * kTile + lane);
        }
        if (step == 5) mask1 = tile_mask(a, u, pn1, row1);
        if (step >= kCopyFirst && (step - kCopyFirst) % kCopyEvery == 0 &&
            (step - kCopyFirst) / kCopyEvery < kSteps) {
          if constexpr (kKv8)
            copy_step8_at(next_copy8, (step - kCopyFirst) / kCopyEvery, std::make_integer_sequence<int, kCopySteps8>());
          else
            copy_step_at(next_copy, (step - kCopyFirst) / kCopyEvery, std::make_integer_sequence<int, kCopySteps>());
        }
      };

      const char LDS_AS *tb = (const char LDS_AS *)(sm.tile[kKv8 ? 1 : cur]);

#pragma unroll
      for (int sb = 0; sb < kSubBlocks; ++sb) {
        // Token half of this score block: the sub-block (128 rows) or the
        // wave's own half (64 rows, where th is already in k_base).
        const int tok = kRows == 128 ? sb : th;
        // ---- scores S^T = K . Q^T for 32 tokens and the wave's 32 rows.  The
        // operand of step st + kKAhead is read while step st multiplies.
        f32x16 s;
        {
          bf16x8 kr[kKAhead + 1];
          auto k_read = [&](int st) {
            return *(const bf16x8 LDS_AS *)(tb + (k_base ^ ((st & 3) << 5)) + (st >> 2) * kGroupBytes +
                                             (kRows == 128 ? sb * 32 * 128 : 0));
          };
#pragma unroll
          for (int st = 0; st < kKAhead; ++st) kr[st] = k_read(st);
#pragma unroll
          for (int st = 0; st < kQkSteps; ++st) {
            tile_step_work(sb * kQkSteps + st);
            if (st + kKAhead < kQkSteps) kr[(st + kKAhead) % (kKAhead + 1)] = k_read(st + kKAhead);
            // (The int8 kernels run at the register limit, where the allocator
            // parks query operands in AGPRs: their MFMAs carry the guard.)
            if (st == 0)
              mfma_vgpr_first<kKv8>(s, kr[0], qr[0]);
            else
              mfma_vgpr<kKv8>(s, kr[st % (kKAhead + 1)], qr[st]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        mfma_result_fence(s);

        // ---- mask, weights.  Register r of lane (n, half) is token
        // 32 tok + 8 (r / 4) + 4 half + r % 4 of the tile.  Scores stay unscaled
        // until the exponent (the scale is positive, so the maximum commutes).
        float x[16];
        float sg[16], sgi[16];  // int8 cache: row factors of the lane's 16 tokens, and inverses
        if constexpr (kKv8) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 v4 = *reinterpret_cast<const f32x4 *>(&sm.sig[32 * tok + 8 * i + 4 * half]);
            const f32x4 w4 = *reinterpret_cast<const f32x4 *>(&sm.sig_inv[32 * tok + 8 * i + 4 * half]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              sg[4 * i + j] = v4[j];
              sgi[4 * i + j] = w4[j];
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = sg[r] * (s[r] - q_bias);
        }
        {
          // Whole-vector integer ops: per-element updates of a vector
          // miscompile with this toolchain (every element read element 0).
          const u32x16 tagged = (__builtin_bit_cast(u32x16, s) & ~15u) | kRegIndex;
          s = __builtin_bit_cast(f32x16, tagged);
        }
        if (mask_cur.full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] = s[r];
        } else {
          // Shift once so every bit test uses a compile-time position.
          unsigned long long msk = mask_cur.m[0];
#pragma unroll
          for (int qq = 1; qq < kMaxQPerGroup; ++qq)
            if (q_local == qq) msk = mask_cur.m[qq];
          msk >>= 32 * tok + 4 * half;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int bit = 8 * (r >> 2) + (r & 3);
            x[r] = ((msk >> bit) & 1ull) ? s[r] : -INFINITY;
          }
        }
        // 64-row groups: the block's bookkeeping (block_max) follows the weights.
        bool late = false;
        float smax_l = -INFINITY, smax_o = -INFINITY;  // the lane's and the row's other lane's block maxima
        int id_b = -1;
        // The lane's best token, the row maximum, the reference where this
        // block sets it, and the headroom check (64-row groups).  The weights
        // need only the reference, so wherever it is already fixed (after the
        // first tile of the first pass) this runs after the weights are formed
        // and written: the latency of the two cross-lane reads it uses is then
        // spent on the exponentials instead of being waited out in front of them.
        auto block_max = [&]() {
          if constexpr (kRows == 64) {
            if (smax_l > best_x) {
              best_x = smax_l;
              best_row = id_b;
            }
            const float smax = fmaxf(smax_l, smax_o) * a.scale_log2;
            if (first_pass && t == 0) {
              // The row's reference: the larger first-tile maximum of its two waves.
              if (half == 0) sm.mx[wave][n] = smax;
              lds_barrier();
              m_ref = fmaxf(sm.mx[rh][n], sm.mx[rh + 2][n]);
            }
            overflow |= smax > m_ref + kHeadroomLog2;
          }
        };
        if constexpr (kRows == 128) {
          float smax = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) smax = fmaxf(smax, x[r]);
          {
            // The token of the lane's largest score in this block (register
            // index from the tag): its stream index, looked up at the end (no
            // register to spare in the tile loop of 128-row groups).
            const int rb = (int)(__builtin_bit_cast(unsigned, smax) & 15u);
            const int tok_b = 32 * tok + 8 * (rb >> 2) + 4 * half + (rb & 3);
            const int id_b = t * kTile + tok_b;
            if (smax > best_x) {
              best_x = smax;
              best_row = id_b;
            }
          }
          smax = fmaxf(smax, __shfl_xor(smax, 32)) * a.scale_log2;
          if (m_ref == -INFINITY) m_ref = smax;  // first scores of this row: acc is still 0
          overflow |= smax > m_ref + kHeadroomLog2;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) smax_l = fmaxf(smax_l, x[r]);
          // The token of the lane's largest score in this block (register
          // index from the tag): its cache row, fetched from the lane that
          // holds it.  Both cross-lane reads are issued here.
          const int rb = (int)(__builtin_bit_cast(unsigned, smax_l) & 15u);
          const int tok_b = 32 * tok + 8 * (rb >> 2) + 4 * half + (rb & 3);
          id_b = __shfl(row_cur, tok_b);
          smax_o = __shfl_xor(smax_l, 32);
          late = !(first_pass && t == 0);
          if (!late) block_max();
        }
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[8 * k + e], a.scale_log2, -m_use));
            l_run += pv[e];
            if constexpr (kKv8) pv[e] *= sg[8 * k + e];  // P.V weights carry the row factors
          }
          const u32x4 w = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]),
                           pack_bf16(pv[4], pv[5]), pack_bf16(pv[6], pv[7])};
          // O is normalised by the sum of the bf16 weights the MFMA actually
          // used, so it stays an exact convex combination of the V rows.
#pragma unroll
          for (int e = 0; e < 4; ++e) l_rnd = sum_bf16_pair(l_rnd, w[e], ones2);
          if constexpr (kKv8) {
            // The weights as used, divided by their factors: the softmax weights
            // the P.V product applies to the dequantised rows.
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              l_cvx = __builtin_fmaf(__builtin_bit_cast(float, w[e] << 16), sgi[8 * k + 2 * e], l_cvx);
              l_cvx = __builtin_fmaf(__builtin_bit_cast(float, w[e] & 0xFFFF0000u), sgi[8 * k + 2 * e + 1], l_cvx);
            }
          }
          // P^T operand of k-block 2 tok + k, row tile rh: lane (row n, half)
          // holds tokens 16 (2 tok + k) + 8 (e / 4) + 4 half + e % 4.
          sm.p[2 * tok + k][rh][lane] = __builtin_bit_cast(bf16x8, w);
        }
        if constexpr (kRows == 64) {
          if (late) {
            // (Opaque to the compiler, so that the use of the cross-lane
            // reads, and the wait for them, is not hoisted above the
            // exponentials into code both paths share.)
            asm volatile("" : "+v"(smax_o), "+v"(id_b));
            block_max();
          }
        }
      }
      __syncthreads();  // every wave's weights for this tile are in LDS

      // ---- O^T += V^T . P^T for this wave's 128 columns and all rows, in
      // (k-block kb, column tile ct) steps.  The transposed LDS read gives lane
      // (m, half) V[token(half, e)][col m] for e = 0..3 (rows +0..3) and
      // e = 4..7 (rows +8..11): the k order of P^T.  V operands are read
      // kVAhead steps ahead and each k-block's weights two steps before it.
      {
        constexpr int kVAhead = kRows == 128 ? 1 : 3;  // 4 (128 rows) or 2 MFMAs per V operand
        i16x4 vr[kVAhead + 1][2];
        bf16x8 pr[2][kRowTiles];
        auto v_read = [&](int j, i16x4 *dst) {
          const int kb = j >> 2, ct = j & 3;
          const int grp = (ct >> 1) * kGroupBytes + 16 * kb * 128;
          dst[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)(tb + (v_base ^ ((ct & 1) << 6)) + grp));
          dst[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)(tb + (v_base8 ^ ((ct & 1) << 6)) + grp));
        };
        auto p_read = [&](int kb, bf16x8 *dst) {
#pragma unroll
          for (int rt = 0; rt < kRowTiles; ++rt) dst[rt] = sm.p[kb][rt][lane];
        };
        p_read(0, pr[0]);
#pragma unroll
        for (int j = 0; j < kVAhead; ++j) v_read(j, vr[j]);
#pragma unroll
        for (int j = 0; j < kPvSteps; ++j) {
          const int kb = j >> 2, ct = j & 3;
          tile_step_work(kSubBlocks * kQkSteps + j);
          if (ct == 2 && kb + 1 < 4) p_read(kb + 1, pr[(kb + 1) & 1]);
          if (j + kVAhead < kPvSteps) v_read(j + kVAhead, vr[(j + kVAhead) % (kVAhead + 1)]);
          const i16x4 *v = vr[j % (kVAhead + 1)];
          // Straight from the LDS reads into consecutive registers: no VALU
          // write precedes the MFMA's operand read.
          const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          // (Unguarded: V comes straight from the LDS reads and P from LDS; the
          // hazard scan of the compiled kernels confirms no copy lands in front.)
          for (int rt = 0; rt < kRowTiles; ++rt) mfma_agpr(acc[4 * rt + ct], va, pr[kb & 1][rt]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      mask_cur = mask1;
      if constexpr (kRows == 64) row_cur = row1;
      sig_raw = sig1_raw;
      sig_ok = sig1_ok;
      pn1 = pn2;
      bn1 = bn2;
      pn2 = pn3;
    }

    // ---- recompute vote: did any row outgrow its reference?  With 64 rows
    // each wave also publishes its rows' largest score for the row's other
    // wave.  (The tile buffers are free once every wave is past the last tile
    // and the zero-row copies issued by the last tile have landed.)
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    int *vote = reinterpret_cast<int *>(sm.tile[0]);
    float *seen = reinterpret_cast<float *>(sm.tile[0] + 64);
    if (lane == 0) vote[wave] = __any(overflow) ? 1 : 0;
    // The row's largest score of the pass, base 2 (the scale is positive, so
    // scaling after the maximum is exact).
    const float m_seen = fmaxf(best_x, __shfl_xor(best_x, 32)) * a.scale_log2;
    if (kRows == 64 && half == 0) seen[wave * 32 + n] = m_seen;
    __syncthreads();
    const bool redo = (vote[0] | vote[1] | vote[2] | vote[3]) != 0;
    const float m_all = kRows == 64 ? fmaxf(seen[rh * 32 + n], seen[(rh + 2) * 32 + n]) : m_seen;
    __syncthreads();  // read before the next pass copies into the buffer
    if (!redo) break;
    // Redo the unit with every reference raised to the largest score seen.
    m_ref = m_all;
    first_pass = false;
    start_pass([]() {}, []() {}, []() {});
  }

  // ---- finalize.  Each wave's outputs cover all rows, so the rounded row
  // sums go through LDS (the tile buffers are free now); with 64 rows the sums
  // of a row's two waves are added there too.
  float *l_sh = reinterpret_cast<float *>(sm.tile[0]);  // [sum kind][wave][32]
  const float l_run_w = l_run + __shfl_xor(l_run, 32);
  const float l_rnd_w = l_rnd + __shfl_xor(l_rnd, 32);
  const float l_cvx_w = kKv8 ? l_cvx + __shfl_xor(l_cvx, 32) : 0.f;
  if (half == 0) {
    l_sh[wave * 32 + n] = l_run_w;
    l_sh[kWaves * 32 + wave * 32 + n] = l_rnd_w;
    if constexpr (kKv8) l_sh[2 * kWaves * 32 + wave * 32 + n] = l_cvx_w;
  }
  // Each lane's candidate for the exact-weight step below: the cache row of
  // the token of its largest score this pass and that token's weight p
  // exactly as the softmax step computed it.  [scoring wave][half][row lane].
  int *cand_row = reinterpret_cast<int *>(sm.tile[0] + 2048);
  float *cand_p = reinterpret_cast<float *>(sm.tile[0] + 3072);
  {
    float cp = 0.f;
    if (best_x > -INFINITY) {
      const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
      cp = __builtin_amdgcn_exp2f(__builtin_fmaf(best_x, a.scale_log2, -m_use));
    }
    cand_row[(wave * 2 + half) * 32 + n] = best_x > -INFINITY ? best_row : -1;
    cand_p[(wave * 2 + half) * 32 + n] = cp;
  }
  lds_barrier();
  // Row sum of kind k (0: exact, 1: rounded) of row 32 r_t + n.
  auto row_sum = [&](int k, int r_t) -> float {
    const float *b = l_sh + k * kWaves * 32 + n;
    return kRows == 128 ? b[r_t * 32] : b[r_t * 32] + b[(r_t + 2) * 32];
  };
  if (th == 0 && half == 0 && row_ok) {
    const float l_tot = row_sum(0, rh);
    lbase[out_row(row_local)] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
  acc_result_fence<kAccTiles>(acc);
  // acc[4 rt + ct] register 4 i + j of lane (n, half) is row 32 rt + n, column
  // 128 wave + 32 ct + 8 i + 4 half + j.  Each 32-row tile of the wave's
  // columns is normalised, converted and staged row-major in the wave's slice
  // of the idle second tile buffer, then stored back 16 bytes per lane as
  // whole row segments (4 rows of 256 bytes, or 2 of 512, per instruction)
  // rather than as 16-byte pieces of 32 rows.
  char *stage = sm.tile[1] + wave * 32 * (512 + 16);
  auto store_tile = [&](int rt, auto esz_c) {
    constexpr int kEsz = decltype(esz_c)::value;  // output element bytes
    constexpr int kSeg = 128 * kEsz;              // one row's bytes of this wave's columns
    constexpr int kStride = kSeg + 16;            // padded LDS row pitch
    constexpr int kLanesPerRow = kSeg / 16;
    constexpr int kRowsPerStep = 64 / kLanesPerRow;
#pragma unroll
    for (int k = 0; k < 32 / kRowsPerStep; ++k) {
      const int row = k * kRowsPerStep + lane / kLanesPerRow;
      const int byte = (lane % kLanesPerRow) * 16;
      const u32x4 d = *reinterpret_cast<const u32x4 *>(stage + row * kStride + byte);
      const int rl = 32 * rt + row;
      if (rl < u.rows)
        __builtin_nontemporal_store(
            d, reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(obase) + (out_row(rl) * kDv + 128 * wave) * kEsz + byte));
    }
  };
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    const int r = 32 * rt + n;
    // bf16 cache: normalised by the sum of the rounded weights used.  int8
    // cache: the bias times that sum comes off, then division by the sum of
    // those weights over their factors (an exact convex combination again).
    const bool ok = r < u.rows;
    const int64_t gr = ok ? out_row(r) : 0;
    // This row tile's accumulators as plain floats (the exact-weight step
    // below adds to them; element writes into vectors miscompile).
    float ov[4][16];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const f32x16 t = acc[4 * rt + ct];
#pragma unroll
      for (int e = 0; e < 16; ++e) ov[ct][e] = t[e];
    }
    float l_rnd_row = row_sum(1, rt);
    float l_cvx_row = kKv8 ? row_sum(2, rt) : 0.f;
    // Largest magnitude of the row's unnormalised outputs in this lane's
    // columns (the exact-weight gate below and the fp16 partial scale).
    float omax = 0.f;
    {
      const float cb = kKv8 ? kKv8Bias * l_rnd_row : 0.f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int e = 0; e < 16; ++e) omax = fmaxf(omax, fabsf(ov[ct][e] - cb));
    }
    float omax_fixed = omax;  // before the step's corrections (which add under 2^-9 of a weight)
    // Exact-weight step.  P.V used every weight rounded to bf16 (relative
    // error up to 2^-9).  Where a few tokens carry much of a row's weight and
    // the output is large, that rounding alone moves O by up to 2^-9 |v - O|
    // per token, more than the output's own precision leaves room for.  The
    // row's largest-score token is always among the candidates of its scoring
    // lanes; each candidate holding at least kExactShare of the row's weight,
    // in a row whose output reaches kExactMinOut in the wave's columns, gets
    // the rest of its weight back: O += (p - bf16(p)) v, with the normaliser
    // raised by the same amount (int8 cache: the factor-carrying weight, and
    // that weight over the factor).  Each wave decides for its own 128 columns
    // of the row, so every column stays a convex combination of V rows.
    {
      constexpr int kCands = kRows == 128 ? 2 : 4;
      const float l_exact = row_sum(0, rt);
      const float l0 = kKv8 ? l_cvx_row : l_rnd_row;
      // Decided for the row's 128 columns of this wave, by both lanes that hold
      // them: they share one normaliser (and, for fp16 partials, one scale).
      omax = fmaxf(omax, __shfl_xor(omax, 32));
      const bool big = omax >= kExactMinOut * l0 && l0 > 0.f;
      int crow[kCands];
      float cp[kCands];
      bool need[kCands];
      bool any = false;
#pragma unroll
      for (int k = 0; k < kCands; ++k) {
        const int src = ((rt + 2 * (k >> 1)) * 2 + (k & 1)) * 32 + n;
        crow[k] = cand_row[src];
        cp[k] = cand_p[src];
        need[k] = big && crow[k] >= 0 && cp[k] >= kExactShare * l_exact;
        any |= need[k];
      }
      if (__any(any)) {
        omax_fixed = -1.f;  // recomputed after the corrections
        // Candidates in batches whose loads are all issued before any is used
        // (the 64-row kernels take all four at once; the 128-row kernels,
        // whose tile loop uses every register, one at a time), each loaded
        // word split into scalars at once; rows a lane does not need are not read.
        constexpr int kBatch = kRows == 128 ? 1 : kCands;
        constexpr int kWords = kKv8 ? 16 : 32;
        const int col0 = 128 * wave + 4 * half;
#pragma unroll
        for (int k0 = 0; k0 < kCands; k0 += kBatch) {
          int rowk[kBatch];
          if constexpr (kRows == 128) {
            // 128-row groups keep the stream index: position, block, row.
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
              const int pos = need[k0 + k] ? raw_position<kMode>(a, u, u.i0 + crow[k0 + k]) : 0;
              const int blk = need[k0 + k] ? raw_block(a, u, pos) : 0;
              rowk[k] = blk * a.block_size + (pos & (a.block_size - 1));
            }
          } else {
#pragma unroll
            for (int k = 0; k < kBatch; ++k) rowk[k] = crow[k0 + k];
          }
          unsigned raw[kBatch][kWords];
          float fac[kBatch];
#pragma unroll
          for (int k = 0; k < kBatch; ++k) {
            fac[k] = 1.f;
#pragma unroll
            for (int m = 0; m < kWords; ++m) raw[k][m] = 0u;
            if (need[k0 + k]) {
              if constexpr (kKv8) {
                fac[k] = a.kv_scale[rowk[k]];
                const char *code = reinterpret_cast<const char *>(a.kv) + (int64_t)rowk[k] * kRowBytes8 + col0;
#pragma unroll
                for (int m = 0; m < 16; ++m)
                  raw[k][m] = *reinterpret_cast<const unsigned *>(code + 32 * (m >> 2) + 8 * (m & 3));
              } else {
                const char *vrow = reinterpret_cast<const char *>(a.kv) + (int64_t)rowk[k] * kRowBytes + 2 * col0;
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                  const u32x2 w2 = *reinterpret_cast<const u32x2 *>(vrow + 2 * (32 * (m >> 2) + 8 * (m & 3)));
                  raw[k][2 * m] = w2[0];
                  raw[k][2 * m + 1] = w2[1];
                }
              }
            }
          }
#pragma unroll
          for (int k = 0; k < kBatch; ++k) {
            if (!need[k0 + k]) continue;
            const float pk = cp[k0 + k];
            if constexpr (kKv8) {
              const float fs = fac[k] != 0.f ? fac[k] : 0x1p-100f;
              const float pw = pk * fs;
              const float d = pw - __builtin_bit_cast(float, pack_bf16(pw, 0.f) << 16);
#pragma unroll
              for (int m = 0; m < 16; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  ov[m >> 2][4 * (m & 3) + j] += d * (float)(((raw[k][m] >> (8 * j)) & 255u) ^ 128u);
              l_rnd_row += d;
              l_cvx_row += d * (1.f / fs);
            } else {
              const float d = pk - __builtin_bit_cast(float, pack_bf16(pk, 0.f) << 16);
#pragma unroll
              for (int m = 0; m < 16; ++m) {
                const unsigned lo = raw[k][2 * m], hi = raw[k][2 * m + 1];
                float *dst = &ov[m >> 2][4 * (m & 3)];
                dst[0] += d * __builtin_bit_cast(float, lo << 16);
                dst[1] += d * __builtin_bit_cast(float, lo & 0xFFFF0000u);
                dst[2] += d * __builtin_bit_cast(float, hi << 16);
                dst[3] += d * __builtin_bit_cast(float, hi & 0xFFFF0000u);
              }
              l_rnd_row += d;
            }
          }
        }
      }
    }
    const float l = kKv8 ? l_cvx_row : l_rnd_row;
    const float c0 = kKv8 ? kKv8Bias * l_rnd_row : 0.f;
    auto unbias = [&](float x) { return kKv8 ? x - c0 : x; };
    float mult = l > 0.f ? 1.f / l : 0.f;
    if (okind == kOutFp16) {
      // Scale this row's 128 columns (the two lanes of the row hold them all)
      // so their largest magnitude uses fp16's full range.
      float mx = omax_fixed;
      if (mx < 0.f) {
        mx = 0.f;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(unbias(ov[ct][e])));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float inv_scale;
      mult *= fp16_scale(mx * mult, &inv_scale);
      if (half == 0 && ok) sbase[gr * kWaves + wave] = inv_scale;
    }
    const bool wide_out = okind == kOutFp32;
    const int pitch = wide_out ? 512 + 16 : 256 + 16;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 o = {unbias(ov[ct][4 * i]) * mult, unbias(ov[ct][4 * i + 1]) * mult,
                         unbias(ov[ct][4 * i + 2]) * mult, unbias(ov[ct][4 * i + 3]) * mult};
        const int col = 32 * ct + 8 * i + 4 * half;
        if (wide_out) {
          *reinterpret_cast<f32x4 *>(stage + n * pitch + col * 4) = o;
        } else {
          const u32x2 h = okind == kOutBf16 ? u32x2{pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])}
                                            : u32x2{pack_f16(o[0], o[1]), pack_f16(o[2], o[3])};
          *reinterpret_cast<u32x2 *>(stage + n * pitch + col * 2) = h;
        }
      }
    if (wide_out)
      store_tile(rt, std::integral_constant<int, 4>());
    else
      store_tile(rt, std::integral_constant<int, 2>());
    __builtin_amdgcn_sched_barrier(0);
  }
}

// (O, lse) merge: one wave per (group, row), four rows per work-group.  Every
// lane derives the maximum and the weight sum of the row's n lse values with
// the same fixed-order wave reduction, then owns kCols consecutive columns of
// each 64 * kCols column chunk; partials are summed in index order.
constexpr int kMergeThreads = 256;
constexpr int kMergeRowsPerGroup = kMergeThreads / 64;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = fmaxf(x, __shfl_xor(x, d));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
  return x;
}

// Partial row `part_row`, columns c .. c + kCols - 1, as fp32 (inverse scale folded
// into the weight for fp16 partials).
template <bool kF16, int kCols>
struct PartialCols {
  float v[kCols];
  float scale;
};
template <bool kF16, int kCols>
__device__ __forceinline__ PartialCols<kF16, kCols> load_partial(const MergeArgs &a, int64_t part_row, int c) {
  PartialCols<kF16, kCols> p;
  if constexpr (kF16) {
    static_assert(kCols == 8, "fp16 partials are read 16 bytes at a time");
    p.scale = a.scale_parts[part_row * (a.d_v / 128) + c / 128];
    // Widened one 16-bit half at a time: element access into 16-bit vector
    // types miscompiles with this toolchain (it reused one word for both).
    const u32x4 h = *reinterpret_cast<const u32x4 *>(
        reinterpret_cast<const _Float16 *>(a.o_parts) + part_row * a.d_v + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p.v[2 * e] = half_bits_to_float(h[e] & 0xFFFFu);
      p.v[2 * e + 1] = half_bits_to_float(h[e] >> 16);
    }
  } else {
    p.scale = 1.f;
    const float *src = reinterpret_cast<const float *>(a.o_parts) + part_row * a.d_v + c;
#pragma unroll
    for (int e = 0; e < kCols; e += 4) {
      const f32x4 o = *reinterpret_cast<const f32x4 *>(src + e);
      p.v[e] = o[0];
      p.v[e + 1] = o[1];
      p.v[e + 2] = o[2];
      p.v[e + 3] = o[3];
    }
  }
  return p;
}

template <bool kF16, int kCols>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kMergeRowsPerGroup + (threadIdx.x >> 6);
  const int g = blockIdx.y;
  if (r >= a.rows) return;  // whole wave; no barriers below
  const float *lse = a.lse_parts + (int64_t)g * a.n * a.rows + r;
  // Maximum and weight sum over all n partials; lane j looks at partials j + 64 k.
  float M = -INFINITY, W = 0.f, wl0 = 0.f;
  if (a.n <= 64) {  // one load per lane
    const float li = lane < a.n ? lse[(int64_t)lane * a.rows] : -INFINITY;
    M = wave_max(li);
    wl0 = (M == -INFINITY || li == -INFINITY) ? 0.f : expf(li - M);
    W = wave_sum(wl0);
  } else {
    for (int i = lane; i < a.n; i += 64) M = fmaxf(M, lse[(int64_t)i * a.rows]);
    M = wave_max(M);
    if (M != -INFINITY)
      for (int i = lane; i < a.n; i += 64) {
        const float li = lse[(int64_t)i * a.rows];
        W += li == -INFINITY ? 0.f : expf(li - M);
      }
    W = wave_sum(W);
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  const int64_t out_row = (int64_t)g * a.rows + r;
  const int64_t part0 = (int64_t)g * a.n * a.rows + r;  // partial i's row: part0 + i * rows
  // Every lane runs every column chunk (the weights below live one per lane and
  // are read across lanes); only loads and stores are limited to real columns.
  for (int c0 = 0; c0 < a.d_v; c0 += 64 * kCols) {
    const int c = c0 + lane * kCols;
    const bool cols_ok = c < a.d_v;
    float s[kCols];
#pragma unroll
    for (int e = 0; e < kCols; ++e) s[e] = 0.f;
    // Partials in chunks of 64: lane j holds the weight of partial i0 + j, read
    // back by every lane; sums run in index order, four partials' loads at a time.
    for (int i0 = 0; i0 < a.n && M != -INFINITY; i0 += 64) {
      const int cnt = min(64, a.n - i0);
      float wl = wl0;
      if (a.n > 64) {
        wl = 0.f;
        if (lane < cnt) {
          const float li = lse[(int64_t)(i0 + lane) * a.rows];
          wl = li == -INFINITY ? 0.f : expf(li - M);
        }
      }
      if (!cols_ok) continue;
      int i = 0;
      for (; i + 4 <= cnt; i += 4) {
        PartialCols<kF16, kCols> p[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) p[k] = load_partial<kF16, kCols>(a, part0 + (int64_t)(i0 + i + k) * a.rows, c);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float wi =
              __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), i + k)) * p[k].scale;
#pragma unroll
          for (int e = 0; e < kCols; ++e) s[e] += wi * p[k].v[e];
        }
      }
      for (; i < cnt; ++i) {
        const PartialCols<kF16, kCols> p = load_partial<kF16, kCols>(a, part0 + (int64_t)(i0 + i) * a.rows, c);
        const float wi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), i)) * p.scale;
#pragma unroll
        for (int e = 0; e < kCols; ++e) s[e] += wi * p.v[e];
      }
    }
    if (cols_ok) {
#pragma unroll
      for (int e = 0; e < kCols; e += 4)
        store_out(a.out, a.out_fp32 ? kOutFp32 : kOutBf16, out_row * a.d_v + c + e,
                  f32x4{s[e] * inv, s[e + 1] * inv, s[e + 2] * inv, s[e + 3] * inv});
    }
  }
  if (lane == 0) a.lse_out[out_row] = W > 0.f ? M + logf(W) : -INFINITY;
}

// Merge of a few partials of 512 columns (the decode's own split-KV merge):
// one wave per row, 8 columns per lane.  Every load (the row's n lse values at
// one address per wave, this lane's columns of each partial and their scale)
// is issued before any is used, so the row costs one memory round trip; every
// lane then forms the maximum, the weights and their sum itself, in index
// order, with no cross-lane traffic.
constexpr int kMergeSmallN = 8;
template <bool kF16, int kN>
__global__ __launch_bounds__(kMergeThreads) void merge_small_kernel(const MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kMergeRowsPerGroup + (threadIdx.x >> 6);
  const int g = blockIdx.y;
  if (r >= a.rows) return;
  const int c = lane * 8;
  const int64_t part0 = (int64_t)g * a.n * a.rows + r;  // partial i's row: part0 + i * rows
  // Raw loads, unconditional (partials past n re-read partial n - 1 and are
  // masked below), so they issue back to back.  Each loaded vector is split
  // into scalars at once: element reads from arrays of vectors miscompile with
  // this toolchain (only element 0 survived).
  float li[kN], sc[kN];
  unsigned raw[kN][kF16 ? 4 : 8];
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    const int64_t pr = part0 + (int64_t)min(i, a.n - 1) * a.rows;
    li[i] = a.lse_parts[pr];
    if constexpr (kF16) {
      sc[i] = a.scale_parts[pr * 4 + (c >> 7)];
      const u32x4 h = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4 *>(reinterpret_cast<const _Float16 *>(a.o_parts) + pr * 512 + c));
#pragma unroll
      for (int e = 0; e < 4; ++e) raw[i][e] = h[e];
    } else {
      sc[i] = 1.f;
      const u32x4 *src = reinterpret_cast<const u32x4 *>(reinterpret_cast<const float *>(a.o_parts) + pr * 512 + c);
      const u32x4 lo = __builtin_nontemporal_load(src), hi = __builtin_nontemporal_load(src + 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        raw[i][e] = lo[e];
        raw[i][4 + e] = hi[e];
      }
    }
  }
  // No branches below (a branch lets the compiler sink the loads after it):
  // partials past n, and partials with lse = -inf, get weight 0.
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kN; ++i) M = fmaxf(M, i < a.n ? li[i] : -INFINITY);
  float W = 0.f;
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.f;
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    const float wi = (i < a.n && li[i] != -INFINITY) ? expf(li[i] - M) : 0.f;
    W += wi;
    const float ws = wi * sc[i];
    float v[8];
    if constexpr (kF16) {
      // Widened one 16-bit half at a time (element access into 16-bit vector
      // types miscompiles with this toolchain).
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = half_bits_to_float(raw[i][e] & 0xFFFFu);
        v[2 * e + 1] = half_bits_to_float(raw[i][e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(float, raw[i][e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += ws * v[e];
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  const int64_t out_row = (int64_t)g * a.rows + r;
  if (a.out_fp32) {
#pragma unroll
    for (int e = 0; e < 8; e += 4)
      store_out(a.out, kOutFp32, out_row * a.d_v + c + e, f32x4{s[e] * inv, s[e + 1] * inv, s[e + 2] * inv, s[e + 3] * inv});
  } else {
    // The lane's 8 bf16 values as one 16-byte store, past the caches (the
    // result is not read again by this call).
    const u32x4 h = {pack_bf16(s[0] * inv, s[1] * inv), pack_bf16(s[2] * inv, s[3] * inv),
                     pack_bf16(s[4] * inv, s[5] * inv), pack_bf16(s[6] * inv, s[7] * inv)};
    __builtin_nontemporal_store(h, reinterpret_cast<u32x4 *>(reinterpret_cast<__bf16 *>(a.out) + out_row * a.d_v + c));
  }
  if (lane == 0) a.lse_out[out_row] = W > 0.f ? M + logf(W) : -INFINITY;
}

// Latent KV-cache write: each wave moves kKvRowsPerWave token rows per pass
// (rows strided over the grid; one row per wave and as many waves as rows, up
// to 32 per CU, measured fastest), loading before storing; lanes move a row's
// 72 chunks of 16 bytes in two passes (64 + 8), so the reads and writes are
// whole 128-byte lines.  Tokens with a negative or out-of-range slot, or (DCP) owned by
// another shard, are skipped.
constexpr int kKvWriteThreads = 256;
constexpr int kKvRowsPerWave = 1;
__global__ __launch_bounds__(kKvWriteThreads) void kv_write_kernel(const KvWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (kKvWriteThreads / 64);
  const int64_t wave0 = (int64_t)blockIdx.x * (kKvWriteThreads / 64) + (threadIdx.x >> 6);
  for (int64_t t0 = wave0; t0 < a.T; t0 += waves * kKvRowsPerWave) {
    u32x4 v[kKvRowsPerWave][2];
    int64_t dst_row[kKvRowsPerWave];
#pragma unroll
    for (int k = 0; k < kKvRowsPerWave; ++k) {
      const int64_t t = t0 + k * waves;
      dst_row[k] = -1;
      if (t < a.T) {
        const int slot = a.slots[t];
        bool store = slot >= 0 && slot < a.num_slots;
        if (a.num_shards > 1) {
          const int p = a.positions[t];
          store = store && p >= 0 && (p / a.interleave) % a.num_shards == a.shard_id;
        }
        if (store) {
          const u32x4 *src = reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(a.rows) + t * kRowBytes);
          v[k][0] = __builtin_nontemporal_load(src + lane);
          if (lane < kChunks - 64) v[k][1] = __builtin_nontemporal_load(src + 64 + lane);
          dst_row[k] = slot;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kKvRowsPerWave; ++k) {
      if (dst_row[k] < 0) continue;  // the whole wave takes the same branch
      u32x4 *dst = reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(a.kv) + dst_row[k] * kRowBytes);
      __builtin_nontemporal_store(v[k][0], dst + lane);
      if (lane < kChunks - 64) __builtin_nontemporal_store(v[k][1], dst + 64 + lane);
    }
  }
}



// ---- Top-k selection of the indexer's scores (the positions a sparse decode
// attends: "vllm-ascend PR #18870 解读：FlashComm1 的'假开启'与 SP 归位", §4.5,
// top-2048 per query token).  Ranking: larger score first, NaN below every
// number, -0 = +0, equal scores by lower position; the chosen positions are
// written in ascending order and the row is padded with -1.
//
// One work-group per row.  Each score maps to a 32-bit key whose unsigned order
// is that ranking (positions break the remaining ties).  The selection finds the
// exact key T of the last chosen element and how many of the keys equal to T to
// take; a last pass marks the keys above T and the keys equal to T in two LDS
// bitmaps (a bit per position); each thread takes one word of each, and one
// block-wide prefix sum of their counts gives every word its output offset (the
// chosen keys above T before it, plus the ties before it up to the number
// taken).  The positions are staged in LDS in order and written out coalesced.
//
// Layout: 1024 threads (16 waves, four per SIMD, so that the many short
// LDS-bound steps of one row overlap); a segment of 32768 positions is 8 slabs
// of 4096, and thread t holds positions 4t .. 4t+3 of every slab (one 16-byte
// load per slab, coalesced across the wave), as keys in registers.
//
// A row of at most one segment (its keys stay in registers) finds T in two
// passes of 16 bits over a histogram of 65536 bins kept as 16-bit counts, two
// to an LDS word (a row has fewer than 65536 keys, so no count carries into its
// neighbour): the first bins the keys by their top half and finds the bin at
// which the count from the top reaches k; the second bins the keys of that bin
// by their low half.  Both add straight from the registers, and only keys at or
// above a lower bound of T take part: each thread's m-th largest key, m =
// ceil(k / 1024), bounds T from below by the smallest of them (at least
// 1024 m >= k keys reach it), which keeps most keys of a typical row out of the
// LDS atomics.  Longer rows are taken segment by segment, reloaded per pass,
// with four passes of one 8-bit digit each.
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkSlabs = 8;                                  // slabs of 4096 positions per segment
constexpr int kTopkSlabLen = 4 * kTopkThreads;
constexpr int kTopkPerThread = 4 * kTopkSlabs;                 // keys held per thread
constexpr int kTopkSeg = kTopkThreads * kTopkPerThread;        // 32768 positions per segment
constexpr int kTopkMapWords = kTopkSeg / 32;                  // bitmap words per segment
constexpr int kTopkMapPerThread = kTopkMapWords / kTopkThreads;  // words of each bitmap a thread takes
static_assert(kTopkMapPerThread >= 1 && kTopkMapPerThread * kTopkThreads == kTopkMapWords, "bitmap split");
constexpr int kTopkMaxM = 4;                                   // largest m the lower bound is formed for
constexpr int kTopkBinWords = 65536 / 2;                       // 16-bit bins, two per LDS word
static_assert(kTopkSeg < 65536, "a bin's count must fit 16 bits");
static_assert(kTopkBinWords >= kTopkWaves * 256 && kTopkBinWords >= kTopkSeg,
              "the histogram's LDS also holds the digit histograms and the staged positions");

__device__ __forceinline__ uint32_t rank_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (x != x) return 1u;          // NaN: below every number (-inf maps to 0x007fffff)
  if ((u << 1) == 0u) u = 0u;     // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The unsigned order of the scores for every value but NaN and -0 (which
// need rank_key): the sign bit set for non-negative values, all bits flipped
// for negative ones.  The mapping is its own inverse up to that choice.
__device__ __forceinline__ uint32_t order_key(uint32_t u) {
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ uint32_t order_key_inverse(uint32_t key) {
  return key ^ ((key & 0x80000000u) ? 0x80000000u : 0xffffffffu);
}
// NaN (either kind) or -0: the scores order_key ranks wrongly.
__device__ __forceinline__ bool needs_rank_key(float x) { return __builtin_amdgcn_classf(x, 0x23); }

// One step of a wave-wide scan through the DPP lane network: lanes that the
// step's source pattern does not reach keep `id`.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_take(uint32_t x, uint32_t id) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, kCtrl, kRowMask, 0xf, false);
}
// Inclusive scan over the 64 lanes of a wave, in registers: shifts by 1, 2, 4
// and 8 lanes inside each row of 16, then the last lane of rows 0 and 2 into
// rows 1 and 3, then the last lane of row 1 into rows 2 and 3.
template <class Op>
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x, uint32_t id, Op op) {
  x = op(x, dpp_take<0x111, 0xf>(x, id));  // row_shr:1
  x = op(x, dpp_take<0x112, 0xf>(x, id));  // row_shr:2
  x = op(x, dpp_take<0x114, 0xf>(x, id));  // row_shr:4
  x = op(x, dpp_take<0x118, 0xf>(x, id));  // row_shr:8
  x = op(x, dpp_take<0x142, 0xa>(x, id));  // row_bcast:15
  x = op(x, dpp_take<0x143, 0xc>(x, id));  // row_bcast:31
  return x;
}
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x, uint32_t id, Op op) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(x, id, op), 63);
}
struct AddU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct MinU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); }
};
struct MaxU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); }
};

// Exclusive prefix sum over the work-group; `total` receives the sum.  The
// trailing barrier frees `part`.
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t *part, uint32_t &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v, 0u, AddU32());
  if (lane == 63) part[wave] = x;
  __syncthreads();
  uint32_t base = 0, sum = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    const uint32_t c = part[i];
    base += i < wave ? c : 0u;
    sum += c;
  }
  __syncthreads();
  total = sum;
  return base + x - v;
}
// The n lowest set bits of x.
__device__ __forceinline__ uint32_t lowest_bits(uint32_t x, uint32_t n) {
  if (n >= (uint32_t)__popc(x)) return x;
  uint32_t r = 0;
  for (uint32_t i = 0; i < n; ++i) {
    r |= x & (0u - x);
    x &= x - 1u;
  }
  return r;
}
// The packed histogram of 16-bit bins: bin b is the low (b even) or high half
// of word b / 2.
__device__ __forceinline__ uint32_t bin_count(const uint32_t *h, uint32_t b) {
  return (h[b >> 1] >> ((b & 1u) << 4)) & 0xffffu;
}
__device__ __forceinline__ void bin_add(uint32_t *h, uint32_t b) { atomicAdd(&h[b >> 1], 1u << ((b & 1u) << 4)); }
// Over the bins wlo .. whi of the packed histogram, the bin at which the count
// from the top first reaches `need` (at least 1 and at most the window's total)
// and the count of the bins above it.  The window is cut into runs of bins from
// the top down; the count above each run comes from a prefix sum over the runs,
// and the run that holds the crossing is walked by one wave, a bin per lane.
// `res` [0, 1] receive the result ([4, 5] are scratch); every thread reads it
// after the last barrier.
__device__ __forceinline__ void crossing_bin(const uint32_t *h, uint32_t wlo, uint32_t whi, uint32_t need,
                                             uint32_t *part, uint32_t *res, uint32_t &bin, uint32_t &above) {
  const uint32_t span = whi > wlo ? whi - wlo : 0u, lane = threadIdx.x & 63;
  // The crossing run (its top bin and the count above it), then the walk.
  auto walk = [&](int64_t run_top, uint32_t per, uint32_t acc0) {
    const int64_t b = run_top - (int64_t)lane;
    const uint32_t c = lane < per && b >= (int64_t)wlo ? bin_count(h, (uint32_t)b) : 0u;
    const uint32_t incl = wave_inclusive_scan(c, 0u, AddU32());
    const unsigned long long hit = __ballot(acc0 + incl >= need);  // lanes at or past the crossing
    if (lane == (uint32_t)(__ffsll((long long)hit) - 1)) {
      res[0] = (uint32_t)b;
      res[1] = acc0 + incl - c;
    }
  };
  if (span < 64 * 64) {
    // At most 4096 bins: wave 0 alone, runs of at most 64 bins, one per lane.
    if (threadIdx.x < 64) {
      const uint32_t per = span / 64 + 1;
      const int64_t top = (int64_t)whi - (int64_t)lane * per;
      uint32_t s = 0;
      for (uint32_t i = 0; i < per; ++i) {
        const int64_t b = top - i;
        if (b >= (int64_t)wlo) s += bin_count(h, (uint32_t)b);
      }
      const uint32_t incl = wave_inclusive_scan(s, 0u, AddU32()), before = incl - s;
      const unsigned long long hit = __ballot(before < need && need <= incl);
      const uint32_t src = (uint32_t)(__ffsll((long long)hit) - 1);  // the lane whose run holds it
      walk((int64_t)whi - (int64_t)src * per, per, (uint32_t)__builtin_amdgcn_readlane((int)before, (int)src));
    }
  } else {
    // Runs of at most 64 bins, one per thread; the crossing run is handed to wave 0.
    const uint32_t per = span / kTopkThreads + 1;
    const int64_t top = (int64_t)whi - (int64_t)threadIdx.x * per;
    uint32_t s = 0;
    for (uint32_t i = 0; i < per; ++i) {
      const int64_t b = top - i;
      if (b >= (int64_t)wlo) s += bin_count(h, (uint32_t)b);
    }
    uint32_t total;
    const uint32_t before = block_exclusive_sum(s, part, total);
    if (before < need && need <= before + s) {
      res[4] = threadIdx.x;
      res[5] = before;
    }
    __syncthreads();
    if (threadIdx.x < 64) walk((int64_t)whi - (int64_t)res[4] * per, per, res[5]);
  }
  __syncthreads();
  bin = res[0];
  above = res[1];
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const TopkArgs a) {
  // the packed 16-bit histogram; also the per-wave digit histograms of long
  // rows, and the staged positions once T is known
  __shared__ __attribute__((aligned(16))) uint32_t h32[kTopkBinWords];
  __shared__ uint32_t gt_map[kTopkMapWords], eq_map[kTopkMapWords];
  __shared__ uint32_t total[256];
  __shared__ uint32_t part[kTopkWaves];
  __shared__ uint32_t pick[2][2];  // per pass parity: chosen digit, count of keys above it
  __shared__ uint32_t res[6];      // crossing bin and count above it; low-half min and max; scratch
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  const int b = row / a.Q, q = row % a.Q;
  const float *src = a.scores + (int64_t)b * a.stride_b + (int64_t)q * a.stride_q;
  int32_t *dst = a.out + (int64_t)row * a.top_k;
  const int L = min(max(a.seq_lens[b] - a.Q + q + 1, 0), a.max_len);
  const int k = min(a.top_k, L);
  for (int i = k + tid; i < a.top_k; i += kTopkThreads) dst[i] = -1;
  if (k == L) {  // every position is chosen
    for (int i = tid; i < L; i += kTopkThreads) dst[i] = i;
    return;
  }
  // key 0 = past the row: below every score (whose keys are >= 1).  Every
  // load is issued unconditionally from a clamped address and the keys of
  // positions past the row are set afterwards, so all loads of a segment are in
  // flight together: 16-byte loads when the row is 16-byte aligned and a
  // multiple of 4 long (a load then never straddles the row's end), else
  // 4-byte loads.
  const bool vec = (reinterpret_cast<uintptr_t>(src) & 15) == 0 && (L & 3) == 0;
  const bool resident = L <= kTopkSeg;
  uint32_t key[kTopkPerThread];
  // Keys come from order_key; a lane that loaded a NaN or a -0 redoes its keys
  // with rank_key (rare, so the common path skips it).
  uint32_t low_or = 0;  // the loaded scores' low 16 bits, OR-ed (nonzero also after a NaN or -0)
  auto load = [&](int seg) {
    bool special = false;
    if (vec) {
      u32x4 f[kTopkSlabs];
#pragma unroll
      for (int j = 0; j < kTopkSlabs; ++j)
        f[j] = *reinterpret_cast<const u32x4 *>(src + min(seg + kTopkSlabLen * j + 4 * tid, L - 4));
#pragma unroll
      for (int j = 0; j < kTopkSlabs; ++j) {
        // keeps the compiler from merging this branch into the 4-byte one
        // (whose key arithmetic is the same) and splitting the 16-byte loads
        asm volatile("" : "+v"(f[j]));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          key[4 * j + c] = order_key(f[j][c]);
          special |= needs_rank_key(__uint_as_float(f[j][c]));
          low_or |= f[j][c] & 0xffffu;
        }
      }
    } else {
      float f[kTopkPerThread];
#pragma unroll
      for (int j = 0; j < kTopkPerThread; ++j)
        f[j] = src[min(seg + kTopkSlabLen * (j >> 2) + 4 * tid + (j & 3), L - 1)];
#pragma unroll
      for (int j = 0; j < kTopkPerThread; ++j) {
        key[j] = order_key(__float_as_uint(f[j]));
        special |= needs_rank_key(f[j]);
        low_or |= __float_as_uint(f[j]) & 0xffffu;
      }
    }
    if (special) {
      low_or = 1u;
#pragma unroll
      for (int j = 0; j < kTopkPerThread; ++j) key[j] = rank_key(__uint_as_float(order_key_inverse(key[j])));
    }
    if (seg + kTopkSeg > L) {  // the row ends in this segment: key 0 past it
      const int rem = L - seg - 4 * tid;  // this thread's key j is in the row iff its offset is below rem
#pragma unroll
      for (int j = 0; j < kTopkPerThread; ++j)
        key[j] = kTopkSlabLen * (j >> 2) + (j & 3) < rem ? key[j] : 0u;
    }
  };
  if (resident) {
    // clear the histogram (its words are first used after the lower bound's
    // barrier), then load the row
#pragma unroll
    for (int i = 0; i < kTopkBinWords / 4 / kTopkThreads; ++i)
      reinterpret_cast<u32x4 *>(h32)[tid + i * kTopkThreads] = u32x4{0u, 0u, 0u, 0u};
    load(0);
  }

  // Lower bound of T (keys below it are never counted) and the largest key.
  uint32_t lo = 1u, hi = 0xffffffffu;
  bool wide_keys = true;  // some score of the row has nonzero low 16 bits (or is NaN / -0)
  const int m = (k + kTopkThreads - 1) / kTopkThreads;
  if (resident && m <= kTopkMaxM) {
    // This thread's m largest keys, descending (an insertion network m deep).
    uint32_t t[kTopkMaxM] = {0u, 0u, 0u, 0u};
    auto largest = [&](auto depth) {
      constexpr int kDepth = decltype(depth)::value;
#pragma unroll
      for (int j = 0; j < kTopkPerThread; ++j) {
        uint32_t x = key[j];
        if constexpr (kDepth == 2) {  // t0 >= t1: the new second largest is the median
          t[1] = max(t[1], min(t[0], x));
          t[0] = max(t[0], x);
        } else {
#pragma unroll
          for (int r = 0; r < kDepth; ++r) {
            const uint32_t hi = max(t[r], x);
            x = min(t[r], x);
            t[r] = hi;
          }
        }
      }
    };
    if (m == 1) largest(std::integral_constant<int, 1>());
    else if (m == 2) largest(std::integral_constant<int, 2>());
    else if (m == 3) largest(std::integral_constant<int, 3>());
    else largest(std::integral_constant<int, 4>());
    const uint32_t mth = m == 1 ? t[0] : m == 2 ? t[1] : m == 3 ? t[2] : t[3];
    // threads with fewer than m keys (mth == 0) do not take part
    const uint32_t mn = wave_reduce(mth ? mth : 0xffffffffu, 0xffffffffu, MinU32());
    const uint32_t cnt = wave_reduce(mth ? 1u : 0u, 0u, AddU32());
    const uint32_t mx = wave_reduce(t[0], 0u, MaxU32());
    const uint32_t wl = wave_reduce(low_or, 0u, [](uint32_t x, uint32_t y) { return x | y; });
    if (lane == 0) {
      total[wave] = mn;
      total[kTopkWaves + wave] = cnt;
      total[2 * kTopkWaves + wave] = mx;
      total[3 * kTopkWaves + wave] = wl;
    }
    __syncthreads();
    // The scheduling fences at the phase boundaries of this kernel keep the
    // compiler from moving work across them (measured: without them a call
    // takes about 2 us longer).
    __builtin_amdgcn_sched_barrier(0);
    uint32_t bmin = 0xffffffffu, bcnt = 0, bmax = 0, bl = 0;
#pragma unroll
    for (int i = 0; i < kTopkWaves; ++i) {
      bmin = min(bmin, total[i]);
      bcnt += total[kTopkWaves + i];
      bmax = max(bmax, total[2 * kTopkWaves + i]);
      bl |= total[3 * kTopkWaves + i];
    }
    wide_keys = bl != 0;
    __syncthreads();
    if (bcnt * (uint32_t)m >= (uint32_t)k) lo = bmin;
    hi = bmax;
  }

  uint32_t prefix = 0, remaining = (uint32_t)k;
  if (resident) {
    if (m > kTopkMaxM) __syncthreads();  // the cleared histogram (else the lower bound's barriers order it)
    // Top halves of the keys at or above lo: the bin of T and the count above it.
#pragma unroll
    for (int j = 0; j < kTopkPerThread; ++j)
      if (key[j] >= lo) bin_add(h32, key[j] >> 16);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    uint32_t b1, above1;
    crossing_bin(h32, lo >> 16, hi >> 16, (uint32_t)k, part, res, b1, above1);
    __builtin_amdgcn_sched_barrier(0);
    if (!wide_keys) {
      // Every score is a bf16 value: all keys of a bin are equal (low half 0
      // for non-negative scores, all ones for negative ones), so the bin
      // gives T.
      prefix = (b1 << 16) | ((b1 & 0x8000u) ? 0u : 0xffffu);
      remaining = (uint32_t)k - above1;
      __builtin_amdgcn_sched_barrier(0);
    } else {
      // Only the bins lo .. hi were counted into: clear their words again.
      for (uint32_t w = (lo >> 17) + (uint32_t)tid; w <= (hi >> 17); w += kTopkThreads) h32[w] = 0u;
      if (tid == 0) {
        res[2] = 0xffffu;
        res[3] = 0u;
      }
      __syncthreads();
      // Low halves of the counted keys in that bin, and their range.
#pragma unroll
      for (int j = 0; j < kTopkPerThread; ++j) {
        const uint32_t kk = key[j];
        if (kk >= lo && (kk >> 16) == b1) {
          const uint32_t l = kk & 0xffffu;
          bin_add(h32, l);
          // a per-lane address: plain LDS atomics rather than a wave-wide
          // reduction loop in each of the 32 unrolled copies
          uint32_t z;
          asm volatile("v_mov_b32 %0, 0" : "=v"(z));
          atomicMin(&res[2] + z, l);
          atomicMax(&res[3] + z, l);
        }
      }
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      uint32_t b2, above2;
      crossing_bin(h32, res[2], res[3], (uint32_t)k - above1, part, res, b2, above2);
      prefix = (b1 << 16) | b2;
      remaining = (uint32_t)k - above1 - above2;
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // Four 8-bit digits from the top, each histogrammed per wave over the keys
    // that match the digits chosen so far.
    uint32_t(*hist)[256] = reinterpret_cast<uint32_t(*)[256]>(h32);
#pragma unroll
    for (int i = 0; i < kTopkWaves * 256 / kTopkThreads; ++i) (&hist[0][0])[tid + i * kTopkThreads] = 0u;
    __syncthreads();
    uint32_t mask = 0;
    for (int shift = 24, pass = 0; shift >= 0; shift -= 8, ++pass) {
      // hist[] is zero here (cleared where it was last summed)
      for (int seg = 0; seg < L; seg += kTopkSeg) {
        load(seg);
#pragma unroll
        for (int j = 0; j < kTopkPerThread; ++j) {
          const uint32_t kk = key[j];
          if (kk != 0u && (kk & mask) == prefix) atomicAdd(&hist[wave][(kk >> shift) & 255u], 1u);
        }
      }
      __syncthreads();
      if (tid < 256) {
        uint32_t t = 0;
#pragma unroll
        for (int c = 0; c < kTopkWaves; ++c) {
          t += hist[c][tid];
          hist[c][tid] = 0u;
        }
        total[tid] = t;
      }
      __syncthreads();
      if (wave == 0) {
        // Lane l owns digits 4l .. 4l+3.  Count above its digits = the sum over
        // higher lanes; then walk its own digits downwards.
        uint32_t c[4], own = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = total[4 * lane + j];
          own += c[j];
        }
        uint32_t x = own;  // inclusive sum from the top lane down
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t y = __shfl_down(x, o, 64);
          if (lane + o < 64) x += y;
        }
        uint32_t above = x - own;
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          if (above < remaining && remaining <= above + c[j]) {
            pick[pass & 1][0] = (uint32_t)(4 * lane + j);
            pick[pass & 1][1] = above;
          }
          above += c[j];
        }
      }
      __syncthreads();
      prefix |= pick[pass & 1][0] << shift;
      mask |= 255u << shift;
      remaining -= pick[pass & 1][1];
    }
  }
  // prefix is now the key T of the last element chosen; `remaining` of the keys
  // equal to T are taken, lowest positions first.
  const bool staged = k <= kTopkSeg;  // positions staged in LDS (the lists are done)
  uint32_t *stage = h32;
  uint32_t above_seen = 0, equal_seen = 0;
  for (int seg = 0; seg < L; seg += kTopkSeg) {
    if (!resident) load(seg);
#pragma unroll
    for (int i = 0; i < kTopkMapWords / kTopkThreads; ++i) {
      gt_map[tid + i * kTopkThreads] = 0u;
      eq_map[tid + i * kTopkThreads] = 0u;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTopkSlabs; ++j) {
      uint32_t g = 0, e = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        g |= (uint32_t)(key[4 * j + c] > prefix) << c;
        e |= (uint32_t)(key[4 * j + c] == prefix) << c;
      }
      const int w = (kTopkSlabLen * j + 4 * tid) >> 5, sh = (4 * tid) & 31;
      if (g) atomicOr(&gt_map[w], g << sh);
      if (e) atomicOr(&eq_map[w], e << sh);
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    const int w0 = kTopkMapPerThread * tid;
    uint32_t gw[kTopkMapPerThread], ew[kTopkMapPerThread];
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int h = 0; h < kTopkMapPerThread; ++h) {
      gw[h] = gt_map[w0 + h];
      ew[h] = eq_map[w0 + h];
      cg += __popc(gw[h]);
      ce += __popc(ew[h]);
    }
    uint32_t sums;
    const uint32_t before = block_exclusive_sum(cg | (ce << 16), part, sums);
    uint32_t above_before = above_seen + (before & 0xffffu), eq_before = equal_seen + (before >> 16);
#pragma unroll
    for (int h = 0; h < kTopkMapPerThread; ++h) {
      const uint32_t g = gw[h], e = ew[h];
      const uint32_t take = remaining > eq_before ? remaining - eq_before : 0u;
      uint32_t sel = g | lowest_bits(e, take);
      uint32_t o = above_before + min(eq_before, remaining);
      const int p0 = seg + 32 * (w0 + h);
      while (sel) {
        const int bit = __ffs(sel) - 1;
        if (o < (uint32_t)k) {
          if (staged) stage[o] = p0 + bit;
          else dst[o] = p0 + bit;
        }
        ++o;
        sel &= sel - 1u;
      }
      above_before += __popc(g);
      eq_before += __popc(e);
    }
    __builtin_amdgcn_sched_barrier(0);
    above_seen += sums & 0xffffu;
    equal_seen += sums >> 16;
    __syncthreads();  // the bitmaps are cleared for the next segment
  }
  __builtin_amdgcn_sched_barrier(0);
  if (staged)
    for (int i = tid; i < k; i += kTopkThreads) dst[i] = stage[i];
}

}  // namespace

hipError_t scratch_buffer(void **ptr, size_t *bytes) {
  // The address of each device's copy, looked up the first time a call runs
  // on that device (with it current), then reused.
  constexpr int kMaxDevices = 64;
  static void *addr[kMaxDevices] = {};
  static std::mutex mu;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs &args, int64_t grid, hipStream_t stream) {
  const dim3 g((unsigned)grid), b(kThreads);
  const bool wide = args.kernel_rows == 128;
  if (args.kv8) {
    if (wide) return hipErrorInvalidValue;  // the planner never picks 128 rows for int8
    if (args.sparse) hipLaunchKernelGGL((decode_kernel<kSparseStream, 64, true>), g, b, 0, stream, args);
    else if (args.num_shards > 1) hipLaunchKernelGGL((decode_kernel<kShardStream, 64, true>), g, b, 0, stream, args);
    else hipLaunchKernelGGL((decode_kernel<kDenseStream, 64, true>), g, b, 0, stream, args);
  } else if (args.sparse) {
    if (wide) hipLaunchKernelGGL((decode_kernel<kSparseStream, 128>), g, b, 0, stream, args);
    else hipLaunchKernelGGL((decode_kernel<kSparseStream, 64>), g, b, 0, stream, args);
  } else if (args.num_shards > 1) {
    if (wide) hipLaunchKernelGGL((decode_kernel<kShardStream, 128>), g, b, 0, stream, args);
    else hipLaunchKernelGGL((decode_kernel<kShardStream, 64>), g, b, 0, stream, args);
  } else {
    if (wide) hipLaunchKernelGGL((decode_kernel<kDenseStream, 128>), g, b, 0, stream, args);
    else hipLaunchKernelGGL((decode_kernel<kDenseStream, 64>), g, b, 0, stream, args);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &args, hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)((int64_t)args.B * args.Q)), dim3(kTopkThreads), 0, stream,
                     args);
  return hipGetLastError();
}

hipError_t launch_kv_write(const KvWriteArgs &args, hipStream_t stream) {
  // Enough waves to keep every CU's memory pipeline busy; each strides over rows.
  const int64_t rows_per_block = kKvWriteThreads / 64 * kKvRowsPerWave;
  const int64_t blocks = std::min<int64_t>((args.T + rows_per_block - 1) / rows_per_block, 256 * 32);
  hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)blocks), dim3(kKvWriteThreads), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs &args, hipStream_t stream) {
  const dim3 grid((unsigned)((args.rows + kMergeRowsPerGroup - 1) / kMergeRowsPerGroup), (unsigned)args.groups);
  if (args.d_v == 512 && args.n <= kMergeSmallN) {
    // The kernel loads kN partials unconditionally: take the smallest kN >= n.
    const dim3 b(kMergeThreads);
    if (args.f16) {
      if (args.n <= 2) hipLaunchKernelGGL((merge_small_kernel<true, 2>), grid, b, 0, stream, args);
      else if (args.n <= 4) hipLaunchKernelGGL((merge_small_kernel<true, 4>), grid, b, 0, stream, args);
      else hipLaunchKernelGGL((merge_small_kernel<true, 8>), grid, b, 0, stream, args);
    } else {
      if (args.n <= 2) hipLaunchKernelGGL((merge_small_kernel<false, 2>), grid, b, 0, stream, args);
      else if (args.n <= 4) hipLaunchKernelGGL((merge_small_kernel<false, 4>), grid, b, 0, stream, args);
      else hipLaunchKernelGGL((merge_small_kernel<false, 8>), grid, b, 0, stream, args);
    }
  } else if (args.f16) {
    if (args.d_v % 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL((merge_kernel<true, 8>), grid, dim3(kMergeThreads), 0, stream, args);
  } else if (args.d_v % 8 == 0) {
    hipLaunchKernelGGL((merge_kernel<false, 8>), grid, dim3(kMergeThreads), 0, stream, args);
  } else {
    hipLaunchKernelGGL((merge_kernel<false, 4>), grid, dim3(kMergeThreads), 0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace mla
