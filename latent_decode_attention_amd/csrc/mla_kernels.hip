// MLA decode attention kernels for gfx950 (MI355X).
//
// One work-group (4 waves x 64 lanes) owns one (sequence, query-token group,
// shard, KV partition) unit and streams that unit's latent rows through LDS in
// 64-token tiles.  Every query head of the group dots the same latent row
// (h_kv = 1 for MLA: "RFC: MsModeling 支持 Decode Context Parallel 仿真",
// §2.1.4 symbol table), so per tile the work is two dense contractions that
// run on the bf16 matrix cores:
//   S^T[token, head] = K_tile[64 x 576] . Q^T[576 x 32]        (per wave)
//   O^T[col, head]  += V_tile^T[512 x 64] . P^T[64 x 32]        (per wave)
// with V_tile = the first 512 columns of the same LDS rows.  The softmax is
// the online (running max / running sum) form; the KV partitions of one unit
// and the DCP shards are combined by the same log-sum-exp merge the DCP page
// describes (§1.1, §2.1.4.3).
//
// Data movement:
//  * the block-table lookup (§2.1.4.1, table A) of tile t+2 and the sparse
//    index load of tile t+3 are issued while tile t is being computed;
//  * tile t+1 is copied HBM -> LDS with direct-to-LDS 16-byte loads
//    (global_load_lds_dwordx4) while tile t is being computed; positions that
//    are padding, out of range or beyond the causal limit are zero-filled in
//    LDS and never read from memory;
//  * an LDS tile holds 64 rows as 9 column groups of 128 bytes (8 chunks of
//    16 bytes): group g of row r lives at g * 8192 + r * 128.  Within a group
//    the chunks of row r are XOR-swizzled by a key of r mod 8 so that the K
//    reads (8 rows, same chunk) and the transposed V reads (4 rows, two
//    neighbouring chunks) each hit 32 distinct banks, and so that each lane's
//    direct loads come from only two rows.
#include <hip/hip_runtime.h>
#include <math.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowBytes = kDqk * 2;                           // 1152
constexpr int kChunks = kRowBytes / 16;                       // 72
constexpr int kTileBytes = kTile * kRowBytes;                 // 73728
constexpr int kQkSteps = kDqk / 16;                           // 36 k-steps of the 32x32x16 MFMA
constexpr int kGroups = kChunks / 8;                          // 9 column groups of 128 bytes
constexpr int kGroupBytes = kTile * 128;                      // 8192
constexpr int kColTiles = kDv / 32;                           // 16 output column tiles
// How far (base 2) a score may exceed its row's reference maximum before the
// unit is recomputed with a higher reference: p <= 2^60 keeps sum(p) * |v| far
// inside the fp32 range for any realistic row.
constexpr float kHeadroomLog2 = 60.0f;
constexpr unsigned kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0), other counters unconstrained

static_assert(kTile == 16 * kWaves, "each wave copies 16 rows of a tile");

struct __attribute__((aligned(16))) Smem {
  char tile[2][kTileBytes];                   // double-buffered latent rows
  int32_t row[2][kTile];                      // physical row per tile token, -1 = not loaded
  unsigned long long mask[3][kMaxQPerGroup];  // attended-token bitmask per query token
  int32_t restarts;                           // bumped when a row needs a higher reference
};


// ---- Matrix-core helpers.  The 256 output accumulators of a lane fill the
// whole AGPR file, so the MFMAs are written as inline asm with register-class
// constraints (scores in VGPRs, outputs in AGPRs) to keep the allocator from
// shuffling them.  Hazards the compiler cannot see through the asm are covered
// by the fences below (s_nop counts exceed the 8-pass 32x32x16 MFMA's needs).
__device__ __forceinline__ void mfma_vgpr_first(f32x16 &d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr(f32x16 &d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_agpr(f32x16 &d, bf16x8 a, bf16x8 b) {
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
__device__ __forceinline__ void valu_result_fence(bf16x8 &a, bf16x8 &b) {
  asm volatile("s_nop 3" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void acc_result_fence(f32x16 *acc) {
  asm volatile("s_nop 15\n\ts_nop 3" ::: "memory");
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) asm volatile("" : "+a"(acc[ct]));
}

__device__ __forceinline__ int chunk_key(int row) {
  const int x = row & 7;
  return ((x & 3) << 1) | (x >> 2);
}

// Byte offset in a tile of logical 16-byte chunk `lc` of tile row `r`.
__device__ __forceinline__ int chunk_off(int r, int lc) {
  return (lc >> 3) * kGroupBytes + r * 128 + (((lc ^ chunk_key(r)) & 7) << 4);
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
  int S, i0, i1;
  int64_t idx_base;
};

template <int kMode>
__device__ __forceinline__ Unit decode_unit(const DecodeArgs &a) {
  const int64_t grid = (int64_t)gridDim.x;
  int64_t id = blockIdx.x;
  // Work-groups are dealt round-robin to the 8 XCDs; renumber so that the
  // partitions of one unit (which share the unit's query rows) sit on one XCD.
  if ((grid & 7) == 0) id = (id & 7) * (grid >> 3) + (id >> 3);
  Unit u;
  u.split = (int)(id % a.splits);
  id /= a.splits;
  const int qg = (int)(id % a.q_groups);
  id /= a.q_groups;
  const int su = (int)(id % a.shard_units);
  u.b = (int)(id / a.shard_units);
  u.q0 = qg * a.q_per_group;
  u.shard = a.shard_base + su;
  u.S = a.seq_lens[u.b];
  int L;
  if constexpr (kMode == kSparseStream)
    L = a.top_k;
  else if constexpr (kMode == kShardStream)
    L = shard_len(u.S, a.num_shards, a.interleave, u.shard);
  else
    L = u.S > 0 ? u.S : 0;
  u.i0 = u.split * a.chunk;
  u.i1 = min(L, u.i0 + a.chunk);
  u.idx_base = kMode == kSparseStream ? (int64_t)u.b * a.idx_stride_b + (int64_t)u.q0 * a.idx_stride_q : 0;
  return u;
}

// Logical token position of stream index i (dense: the position itself or the
// i-th position owned by the shard; sparse: the i-th list entry).  -1 past the end.
template <int kMode>
__device__ __forceinline__ int stream_position(const DecodeArgs &a, const Unit &u, int i) {
  if (i >= u.i1) return -1;
  if constexpr (kMode == kSparseStream) return a.indices[u.idx_base + i];
  if constexpr (kMode == kShardStream)
    return ((i / a.interleave) * a.num_shards + u.shard) * a.interleave + (i % a.interleave);
  return i;
}

// Block-table entry for position p, or -1 when p is never attended by this
// group's query tokens or the entry is out of range.
__device__ __forceinline__ int lookup_block(const DecodeArgs &a, const Unit &u, int p) {
  const int last = u.S - a.Q + u.q0 + a.q_per_group - 1;
  if (p < 0 || p > last) return -1;
  const int slot = p >> a.bs_shift;
  if (slot >= a.max_blocks) return -1;
  const int blk = a.block_table[(int64_t)u.b * a.max_blocks + slot];
  return (blk >= 0 && blk < a.num_blocks) ? blk : -1;
}

// Prefetch variants used inside the tile loop: the loads are unconditional with
// clamped (always in-bounds) addresses and their values are only examined after
// the tile's math, so no wait on them lands in front of the math (a wait there
// would also drain the in-flight copy of the next tile).
__device__ __forceinline__ int raw_index(const DecodeArgs &a, const Unit &u, int i) {
  return a.indices[u.idx_base + min(i, u.i1 - 1)];
}
__device__ __forceinline__ int raw_block(const DecodeArgs &a, const Unit &u, int p) {
  const int slot = min(max(p, 0) >> a.bs_shift, a.max_blocks - 1);
  return a.block_table[(int64_t)u.b * a.max_blocks + slot];
}
__device__ __forceinline__ int checked_block(const DecodeArgs &a, const Unit &u, int p, int raw) {
  const int last = u.S - a.Q + u.q0 + a.q_per_group - 1;
  const bool ok = p >= 0 && p <= last && (p >> a.bs_shift) < a.max_blocks && raw >= 0 &&
                  raw < a.num_blocks;
  return ok ? raw : -1;
}

// Wave 0 publishes the physical rows and attended masks of one tile.
__device__ __forceinline__ void publish_tile(Smem &sm, const DecodeArgs &a, const Unit &u,
                                             int lane, int p, int blk, int row_buf, int mask_buf) {
  const bool ok = blk >= 0;
  sm.row[row_buf][lane] = ok ? blk * a.block_size + (p & (a.block_size - 1)) : -1;
  for (int qq = 0; qq < a.q_per_group; ++qq) {
    const unsigned long long m = __ballot(ok && p <= u.S - a.Q + u.q0 + qq);
    if (lane == 0) sm.mask[mask_buf][qq] = m;
  }
}

// One direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at
// LDS address lds_base + 16 l.  The instruction's immediate offset is added to
// both the global and the LDS address, so M0 is pre-biased by it.  Issued as
// inline asm so that the compiler's memory model does not order it against the
// other tile buffer's LDS reads (it would otherwise drain vmcnt before every
// LDS access); completion is awaited explicitly with s_waitcnt vmcnt(0) before
// the barrier that publishes the tile.
// m0 is reserved for the compiler, which uses it for nothing else in these
// kernels; the clobber records that the copy rewrites it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int kOffset>
__device__ __forceinline__ void dma16(const char *src, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off offset:%2"
               :
               : "s"(lds_base - kOffset), "v"(src), "i"(kOffset)
               : "m0");
}
#pragma clang diagnostic pop

template <int G>
__device__ __forceinline__ void dma_row_groups(const char *src, unsigned lds_blk) {
  dma16<G * 128>(src, lds_blk + G * kGroupBytes);
  if constexpr (G + 1 < kGroups) dma_row_groups<G + 1>(src, lds_blk);
}

// All waves: copy one tile of latent rows into LDS buffer `buf`.  Wave w copies
// rows 16w..16w+15; one instruction moves 8 rows x 128 bytes of one column
// group, lane l taking row 16w + 8k + l/8 and stored position l%8 of it.
__device__ __forceinline__ void issue_tile(Smem &sm, const DecodeArgs &a, int buf, int wave, int lane) {
  const char *kvb = reinterpret_cast<const char *>(a.kv);
  const int sub = lane >> 3;                      // row within the 8-row block
  const int lc_lo = (lane & 7) ^ chunk_key(sub);  // logical chunk (mod 8) at this slot
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int r = 16 * wave + 8 * k + sub;
    const int row = sm.row[buf][r];
    const unsigned blk = __builtin_amdgcn_readfirstlane(
        (unsigned)(uintptr_t)(&sm.tile[buf][(16 * wave + 8 * k) * 128]));
    if (row >= 0) {
      dma_row_groups<0>(kvb + (int64_t)row * kRowBytes + lc_lo * 16, blk);
    } else {
#pragma unroll
      for (int g = 0; g < kGroups; ++g)
        *reinterpret_cast<int4 *>(&sm.tile[buf][g * kGroupBytes + (16 * wave + 8 * k) * 128 + lane * 16]) =
            make_int4(0, 0, 0, 0);
    }
  }
}

// Two floats to packed bf16 (round to nearest even, v_cvt_pk_bf16_f32).  Vectors
// of bf16 are only ever assembled from whole 32-bit words: inserting single
// __bf16 elements into a vector miscompiles with this toolchain.
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ __forceinline__ void store_out(void *out, int fp32, int64_t elem, f32x4 v) {
  if (fp32) {
    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + elem) = v;
  } else {
    const u32x2 h = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    *reinterpret_cast<u32x2 *>(reinterpret_cast<__bf16 *>(out) + elem) = h;
  }
}

template <int kMode>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(const DecodeArgs a) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, half = lane >> 5;

  const Unit u = decode_unit<kMode>(a);
  const int ntiles = u.i1 > u.i0 ? (u.i1 - u.i0 + kTile - 1) / kTile : 0;

  // The wave's 32 query rows (q token, head); lane n and n+32 share a row.
  const int row_local = wave * 32 + n;
  const bool row_ok = row_local < a.rows_per_group;
  const int q_local = row_ok ? row_local / a.h_q : 0;
  const int head = row_ok ? row_local - q_local * a.h_q : 0;
  const int64_t grow = ((int64_t)u.b * a.Q + u.q0 + q_local) * a.h_q + head;
  const bool computes = wave * 32 < a.rows_per_group;

  // Output destination: final tensor or this partition's slot of the partials.
  const int64_t su = u.shard - a.shard_base;
  void *obase;
  float *lbase;
  int ofp32;
  if (a.splits > 1) {
    const int64_t g = su * a.splits + u.split;
    obase = a.part_o + g * a.rows_total * kDv;
    lbase = a.part_lse + g * a.rows_total;
    ofp32 = 1;
  } else {
    ofp32 = a.out_fp32;
    obase = ofp32 ? (void *)(reinterpret_cast<float *>(a.out) + su * a.rows_total * kDv)
                  : (void *)(reinterpret_cast<__bf16 *>(a.out) + su * a.rows_total * kDv);
    lbase = a.lse + su * a.rows_total;
  }

  if (ntiles == 0) {
    if (row_ok) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      for (int c = half * 4; c < kDv; c += 8) store_out(obase, ofp32, grow * kDv + c, z);
      if (half == 0) lbase[grow] = -INFINITY;
    }
    return;
  }

  // Query rows in registers: lane (n, half) holds q[row][16 st + 8 half + 0..7], the
  // B operand of the 32x32x16 MFMA for k-step st.
  bf16x8 qr[kQkSteps];
  if (row_ok) {
    const bf16x8 *qp = reinterpret_cast<const bf16x8 *>(a.q + grow * kDqk);
#pragma unroll
    for (int st = 0; st < kQkSteps; ++st) qr[st] = qp[2 * st + half];
  } else {
#pragma unroll
    for (int st = 0; st < kQkSteps; ++st) qr[st] = bf16x8{};
  }

  // Per-lane LDS byte offsets within a tile.  K step st reads logical chunk
  // 2 st + half of row n (+32 for the second sub-block): with the row's XOR key
  // that is column group st / 4 (an immediate) plus one of four per-lane offsets.
  // V step (kb, ct) reads column group ct / 2 (immediate) plus one of two.
  const int key_k = chunk_key(n);
  int k_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) k_off[j] = n * 128 + ((((2 * j + half) ^ key_k) & 7) << 4);
  const int v_row = 4 * half + ((lane & 15) >> 2);    // row within a 16-token k-block
  const int v_key = chunk_key(v_row);
  const int v_lc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // chunk within a 64-byte span
  int v_off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) v_off[j] = v_row * 128 + ((((4 * j + v_lc) ^ v_key) & 7) << 4) + 8 * (lane & 1);
  const bf16x8 zero8 = {};

  // Softmax bookkeeping, base-2 units.  m_ref is the row's reference maximum:
  // set from the first sub-block in which the row attends anything, and only
  // ever raised by a restart.  p = 2^(x - m_ref) may exceed 1 by up to
  // 2^kHeadroom, which fp32 accumulators and bf16 operands carry without loss,
  // so the accumulators are never rescaled inside the loop.
  float m_ref = -INFINITY;
  float m_seen = -INFINITY;  // largest score seen so far
  float l_run = 0.f;         // this lane's share of sum(p), for lse
  float l_rnd = 0.f;         // the same sum over p as rounded to bf16, for O
  f32x16 acc[kColTiles];
  int restarts_seen = 0;

  if (tid == 0) sm.restarts = 0;
  for (;;) {
    // Prologue of a pass: rows and masks of tiles 0 and 1; position of tile 2.
    // (The opaque copy of the lane id keeps this per-pass work from being
    // hoisted out of the restart loop and held in registers.)
    int pf_pos = -1;
    int plane = lane;
    asm volatile("" : "+v"(plane));
    if (wave == 0) {
      const int p0 = stream_position<kMode>(a, u, u.i0 + plane);
      publish_tile(sm, a, u, plane, p0, lookup_block(a, u, p0), 0, 0);
      if (ntiles > 1) {
        const int p1 = stream_position<kMode>(a, u, u.i0 + kTile + plane);
        publish_tile(sm, a, u, plane, p1, lookup_block(a, u, p1), 1, 1);
      }
      if (ntiles > 2) pf_pos = stream_position<kMode>(a, u, u.i0 + 2 * kTile + plane);
    }
    __syncthreads();
    issue_tile(sm, a, 0, wave, lane);

#pragma unroll
    for (int ct = 0; ct < kColTiles; ++ct) acc_zero(acc[ct], zero8);
    l_run = 0.f;
    l_rnd = 0.f;
    bool restart = false;

    for (int t = 0; t < ntiles; ++t) {
      const int cur = t & 1;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's copies of tile t have landed
      __syncthreads();                       // ... and every other wave's
      if (sm.restarts != restarts_seen) {    // uniform: read after the barrier
        restart = true;
        break;
      }
      if (t + 1 < ntiles) issue_tile(sm, a, cur ^ 1, wave, lane);

      // Start the lookups for later tiles so they complete under this tile's math
      // (every wave issues them, only wave 0 uses them).
      const bool pf2 = wave == 0 && t + 2 < ntiles;
      const int i3 = u.i0 + (t + 3) * kTile + lane;
      const int blk2_raw = raw_block(a, u, pf_pos);
      int pos3_raw;
      if constexpr (kMode == kSparseStream)
        pos3_raw = raw_index(a, u, i3);
      else
        pos3_raw = stream_position<kMode>(a, u, i3);

      if (computes) {
        const char LDS_AS *tb = (const char LDS_AS *)(sm.tile[cur]);
        // This lane's tokens are 4 half + {0..3} (+8 i, +32 sb): shift once so
        // every bit test below uses a compile-time position.
        const unsigned long long msk = sm.mask[t % 3][q_local] >> (4 * half);
        bool overflow = false;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          // ---- scores S^T = K . Q^T for the sub-block's 32 tokens.  Operands of
          // step st+2 are read while step st multiplies (3-slot ring); the fences
          // keep the compiler from hoisting every read.
          f32x16 s;
          bf16x8 kr[3];
          auto k_read = [&](int st) {
            return *(const bf16x8 LDS_AS *)(tb + k_off[st & 3] + (st >> 2) * kGroupBytes + sb * 32 * 128);
          };
          kr[0] = k_read(0);
          kr[1] = k_read(1);
#pragma unroll
          for (int st = 0; st < kQkSteps; ++st) {
            if (st + 2 < kQkSteps) kr[(st + 2) % 3] = k_read(st + 2);
            if (st == 0)
              mfma_vgpr_first(s, kr[0], qr[0]);
            else
              mfma_vgpr(s, kr[st % 3], qr[st]);
            __builtin_amdgcn_sched_barrier(0);
          }
          mfma_result_fence(s);

          // ---- mask and scale.  Register r of lane (n, half) is token
          // 8 (r / 4) + 4 half + r % 4 of the sub-block.
          float x[16];
          float smax = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int bit = 32 * sb + 8 * (r >> 2) + (r & 3);
            x[r] = ((msk >> bit) & 1ull) ? s[r] * a.scale_log2 : -INFINITY;
            smax = fmaxf(smax, x[r]);
          }
          smax = fmaxf(smax, __shfl_xor(smax, 32));
          m_seen = fmaxf(m_seen, smax);
          if (m_ref == -INFINITY) m_ref = smax;  // first scores of this row: acc is still 0
          overflow |= smax > m_ref + kHeadroomLog2;
          const float m_use = m_ref == -INFINITY ? 0.f : m_ref;

          bf16x8 pb[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              pv[e] = __builtin_amdgcn_exp2f(x[8 * k + e] - m_use);
              l_run += pv[e];
            }
            const u32x4 w = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]),
                             pack_bf16(pv[4], pv[5]), pack_bf16(pv[6], pv[7])};
            pb[k] = __builtin_bit_cast(bf16x8, w);
            // O is normalised by the sum of the bf16 weights the MFMA actually
            // used, so it stays an exact convex combination of the V rows.
#pragma unroll
            for (int e = 0; e < 4; ++e)
              l_rnd += __builtin_bit_cast(float, w[e] << 16) + __builtin_bit_cast(float, w[e] & 0xFFFF0000u);
          }
          valu_result_fence(pb[0], pb[1]);

          // ---- O^T += V^T . P^T, 16 tokens per MFMA.  The transposed LDS read
          // gives lane (m, half) V[token(half, e)][32 ct + m] for e = 0..3 (rows
          // +0..3) and e = 4..7 (rows +8..11): the k order of P^T above.
          // Step i = 16 kb + ct; operands of step i+2 are read during step i.
          i16x4 vr[3][2];
          auto v_read = [&](int i, i16x4 *dst) {
            const int kb = i >> 4, ct = i & 15;
            const char LDS_AS *va0 = tb + v_off[ct & 1] + (ct >> 1) * kGroupBytes + (32 * sb + 16 * kb) * 128;
            dst[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)va0);
            dst[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS *)(va0 + 8 * 128));
          };
          v_read(0, vr[0]);
          v_read(1, vr[1]);
#pragma unroll
          for (int i = 0; i < 2 * kColTiles; ++i) {
            if (i + 2 < 2 * kColTiles) v_read(i + 2, vr[(i + 2) % 3]);
            const bf16x8 va = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(vr[i % 3][0], vr[i % 3][1], 0, 1, 2, 3, 4, 5, 6, 7));
            mfma_agpr(acc[i & 15], va, pb[i >> 4]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (__any(overflow)) sm.restarts = restarts_seen + 1;
      }

      if (pf2) publish_tile(sm, a, u, lane, pf_pos, checked_block(a, u, pf_pos, blk2_raw), cur, (t + 2) % 3);
      pf_pos = i3 < u.i1 ? pos3_raw : -1;
    }
    if (!restart) {
      __syncthreads();
      restart = sm.restarts != restarts_seen;
    }
    if (!restart) break;
    // Some row's scores outgrew its reference by more than the headroom: redo
    // the unit with every reference raised to the largest score seen.
    ++restarts_seen;
    m_ref = m_seen;
  }

  if (!row_ok) return;
  // The two lanes of a row saw disjoint halves of every tile.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float l_rnd_tot = l_rnd + __shfl_xor(l_rnd, 32);
  const float inv = l_rnd_tot > 0.f ? 1.f / l_rnd_tot : 0.f;
  if (half == 0)
    lbase[grow] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  acc_result_fence(acc);
  // acc[ct] register 4i+j of lane (n, half) is column 32 ct + 8 i + 4 half + j.
#pragma unroll
  for (int ct = 0; ct < kColTiles; ++ct) {
    const f32x16 v = acc[ct];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 o = {v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv};
      store_out(obase, ofp32, grow * kDv + 32 * ct + 8 * i + 4 * half, o);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// (O, lse) merge: one work-group per (group, row); weights in LDS, fixed order.
__global__ __launch_bounds__(128) void merge_kernel(const MergeArgs a) {
  __shared__ float w[1024];
  __shared__ float stats[2];
  const int64_t r = blockIdx.x;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const float *lse = a.lse_parts + (int64_t)g * a.n * a.rows + r;
  if (tid == 0) {
    float M = -INFINITY;
    for (int i = 0; i < a.n; ++i) M = fmaxf(M, lse[(int64_t)i * a.rows]);
    float W = 0.f;
    for (int i = 0; i < a.n; ++i) {
      const float li = lse[(int64_t)i * a.rows];
      const float wi = (M == -INFINITY || li == -INFINITY) ? 0.f : expf(li - M);
      w[i] = wi;
      W += wi;
    }
    stats[0] = M;
    stats[1] = W;
  }
  __syncthreads();
  const float M = stats[0], W = stats[1];
  const float inv = W > 0.f ? 1.f / W : 0.f;
  const int64_t out_row = (int64_t)g * a.rows + r;
  for (int c = tid * 4; c < a.d_v; c += 128 * 4) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < a.n; ++i) {
      if (w[i] == 0.f) continue;
      const f32x4 o = *reinterpret_cast<const f32x4 *>(
          a.o_parts + (((int64_t)g * a.n + i) * a.rows + r) * a.d_v + c);
      s += w[i] * o;
    }
    store_out(a.out, a.out_fp32, out_row * a.d_v + c, s * inv);
  }
  if (tid == 0) a.lse_out[out_row] = W > 0.f ? M + logf(W) : -INFINITY;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &args, int64_t grid, hipStream_t stream) {
  if (args.sparse)
    hipLaunchKernelGGL(decode_kernel<kSparseStream>, dim3((unsigned)grid), dim3(kThreads), 0, stream, args);
  else if (args.num_shards > 1)
    hipLaunchKernelGGL(decode_kernel<kShardStream>, dim3((unsigned)grid), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(decode_kernel<kDenseStream>, dim3((unsigned)grid), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs &args, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)args.rows, (unsigned)args.groups), dim3(128), 0,
                     stream, args);
  return hipGetLastError();
}

}  // namespace mla
