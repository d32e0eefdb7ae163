"""Seeded synthetic inputs for MLA decode over a paged latent KV cache.

This module is shared by the HIP path's tests/benchmark and by the CPU reference;
it therefore holds none of the attention arithmetic: only random draws, their
rounding to bf16, paged block tables and top-k index lists.  Every array is a
numpy array of raw bits (bf16 as uint16) or int32, so that both sides read the
very same bytes.

Shapes follow the symbol table of "RFC: MsModeling 支持 Decode Context Parallel
仿真" (§2.1.4): B sequences, Q query tokens per sequence, h_q heads, one latent
row of D = kv_lora_rank + qk_rope_head_dim = 576 columns per token, stored as
[N_blk, block_size, D] behind a block table (§2.1.4.1, table A).

Recipe (stated once here, used by every config):
  * q and latent rows are fp32 N(0, 1) draws rounded to bf16 (nearest-even);
  * numpy PCG64 seeded per config, with independent SeedSequence children for
    q / cache / block table / indices / outliers;
  * block tables map logical blocks to a seeded random permutation of the
    physical blocks; `spare_blocks` extra physical blocks are filled with NaN
    bit patterns and every table slot a sequence does not use points at one of
    them, so any read of an unused or unreferenced block shows up as NaN;
  * sparse index lists are distinct positions drawn uniformly without
    replacement, sorted ascending, padded with -1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

D_QK = 576          # kv_lora_rank (512) + qk_rope_head_dim (64)
D_V = 512           # latent V = first kv_lora_rank columns
ROPE_COLS = slice(512, 576)
DEFAULT_SCALE = 1.0 / math.sqrt(192.0)
BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One decode problem: inputs as raw bits plus the call parameters."""
    name: str
    B: int
    Q: int
    h_q: int
    scale: float
    block_size: int
    q: np.ndarray            # uint16 [B, Q, h_q, 576]
    kv: np.ndarray           # uint16 [num_blocks, block_size, 576]
    block_table: np.ndarray  # int32 [B, max_blocks]
    seq_lens: np.ndarray     # int32 [B]
    d_qk: int = D_QK
    d_v: int = D_V
    # sparse (top-k) selection; None for dense
    indices: Optional[np.ndarray] = None   # int32, element (b,q,k) at b*stride_b + q*stride_q + k
    top_k: int = 0
    index_stride_b: int = 0
    index_stride_q: int = 0
    # decode-context-parallel sharding (dense); 1 = unsharded
    num_shards: int = 1
    interleave: int = 1
    meta: dict = field(default_factory=dict)
    # int8 latent cache (when set, the cache the workload describes): int8
    # [num_blocks, block_size, 576] and one fp32 factor per row [num_blocks, block_size].
    kv8: Optional[np.ndarray] = None
    kv_scale: Optional[np.ndarray] = None

    @property
    def num_blocks(self) -> int:
        return int(self.kv.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def rows(self) -> int:
        return self.B * self.Q * self.h_q

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())


def _normal_bf16(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """N(0,1) fp32 draws rounded to bf16, generated in bounded chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def make_paged_cache(rng_cache: np.random.Generator, rng_table: np.random.Generator,
                     seq_lens, block_size: int, spare_blocks: int = 8,
                     outlier_rng: Optional[np.random.Generator] = None,
                     outlier_rate: float = 0.0, outlier_factor: float = 8.0):
    """Paged latent cache plus a block table over a seeded permutation of blocks.

    Returns (kv uint16 [num_blocks, block_size, 576], block_table int32 [B, max_blocks]).
    With an outlier rate, a Bernoulli(rate) subset of physical rows gets its
    key-only (RoPE) columns multiplied by `outlier_factor` before rounding.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    nblk = (seq_lens + block_size - 1) // block_size
    used = int(nblk.sum())
    num_blocks = used + spare_blocks
    max_blocks = int(max(1, nblk.max()))
    kv = np.empty((num_blocks, block_size, D_QK), dtype=np.uint16)
    per_block = block_size * D_QK
    flat = kv.reshape(num_blocks, per_block)
    step = max(1, (1 << 24) // per_block)
    for s in range(0, num_blocks, step):
        e = min(num_blocks, s + step)
        x = rng_cache.standard_normal((e - s) * per_block, dtype=np.float32)
        x = x.reshape(e - s, block_size, D_QK)
        if outlier_rng is not None and outlier_rate > 0.0:
            hit = outlier_rng.random((e - s, block_size)) < outlier_rate
            x[:, :, ROPE_COLS] = np.where(hit[:, :, None], x[:, :, ROPE_COLS] * np.float32(outlier_factor),
                                          x[:, :, ROPE_COLS])
        flat[s:e] = f32_to_bf16_bits(x).reshape(e - s, per_block)
    perm = rng_table.permutation(num_blocks)
    phys_used, spares = perm[:used], perm[used:]
    if spare_blocks > 0:
        kv[spares] = BF16_NAN
        filler = int(spares[0])
    else:
        filler = int(phys_used[0]) if used else 0
    bt = np.full((len(seq_lens), max_blocks), filler, dtype=np.int32)
    o = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = phys_used[o:o + n]
        o += n
    return kv, bt


def make_topk_indices(rng: np.random.Generator, seq_lens, top_k: int,
                      short_rows: int = 0, short_valid: int = 0):
    """Sorted distinct positions in [0, S_b) per sequence, -1 padded to top_k.

    min(top_k, S_b) positions are drawn per sequence.  `short_rows` sequences
    (chosen by a seeded permutation) keep only their first `short_valid` sorted
    entries and pad the rest with -1.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = len(seq_lens)
    idx = np.full((B, top_k), -1, dtype=np.int32)
    for b in range(B):
        k = int(min(top_k, seq_lens[b]))
        pick = np.sort(rng.choice(int(seq_lens[b]), size=k, replace=False))
        idx[b, :k] = pick
    if short_rows:
        for b in rng.permutation(B)[:short_rows]:
            idx[b, short_valid:] = -1
    return idx


def _children(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def make_workload(name: str, B: int, Q: int, h_q: int, seq_lens, block_size: int, seed: int,
                  scale: float = DEFAULT_SCALE, top_k: int = 0, shared_q_indices: bool = True,
                  short_rows: int = 0, short_valid: int = 0, num_shards: int = 1,
                  interleave: int = 1, spare_blocks: int = 8, outlier_rate: float = 0.0,
                  outlier_factor: float = 8.0) -> Workload:
    """General seeded workload; the numbered configs below are presets of it."""
    g_q, g_kv, g_bt, g_idx, g_out = _children(seed, 5)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (B,)
    q = _normal_bf16(g_q, (B, Q, h_q, D_QK))
    kv, bt = make_paged_cache(g_kv, g_bt, seq_lens, block_size, spare_blocks,
                              outlier_rng=g_out if outlier_rate > 0 else None,
                              outlier_rate=outlier_rate, outlier_factor=outlier_factor)
    w = Workload(name=name, B=B, Q=Q, h_q=h_q, scale=scale, block_size=block_size, q=q, kv=kv,
                 block_table=bt, seq_lens=seq_lens, num_shards=num_shards, interleave=interleave,
                 meta=dict(seed=seed, short_rows=short_rows, short_valid=short_valid,
                           outlier_rate=outlier_rate))
    if top_k:
        if shared_q_indices:
            idx = make_topk_indices(g_idx, seq_lens, top_k, short_rows, short_valid)
            w.indices, w.index_stride_b, w.index_stride_q = idx, top_k, 0
        else:
            lists = [make_topk_indices(g_idx, seq_lens, top_k, short_rows, short_valid) for _ in range(Q)]
            idx = np.ascontiguousarray(np.stack(lists, axis=1))  # [B, Q, top_k]
            w.indices, w.index_stride_b, w.index_stride_q = idx, Q * top_k, top_k
        w.top_k = top_k
    return w


# ---------------------------------------------------------------------------
# The five decode workloads the method is measured on, plus the dense 32k point.
# ---------------------------------------------------------------------------

def int8_cache(w: Workload) -> Workload:
    """The same workload over an int8 latent cache: each row of the bf16 cache
    becomes int8 codes rint(x / f) with one fp32 factor f = max|x| / 127 per row
    (codes in [-127, 127]; all-zero rows get f = 0).  Rows holding NaN (the
    poisoned spare blocks) get code 0 and factor NaN, so they stay poison.  This
    is an input recipe only: the method reads the codes and factors as given."""
    nb, bs, d = w.kv.shape
    kv8 = np.empty((nb, bs, d), dtype=np.int8)
    fac = np.empty((nb, bs), dtype=np.float32)
    step = max(1, (1 << 22) // (bs * d))
    for s in range(0, nb, step):
        e = min(nb, s + step)
        x = bf16_bits_to_f32(w.kv[s:e])
        bad = np.isnan(x).any(axis=2)
        x = np.where(np.isnan(x), np.float32(0.0), x)
        m = np.abs(x).max(axis=2)
        f = (m / np.float32(127.0)).astype(np.float32)
        safe = np.where(f > 0, f, np.float32(1.0))
        kv8[s:e] = np.clip(np.rint(x / safe[:, :, None]), -127, 127).astype(np.int8)
        fac[s:e] = np.where(bad, np.float32(np.nan), f)
    return replace(w, name=w.name + "_kv8", kv8=kv8, kv_scale=fac)


def config_tiny(seed: int = 1001) -> Workload:
    """Dense, B=1 Q=1 h_q=16 S=256, one contiguous 256-token block."""
    return make_workload("dense_tiny_b1_h16_s256", 1, 1, 16, [256], 256, seed, spare_blocks=0)


def config_dense_paged(seed: int = 1002) -> Workload:
    """Dense, B=32 Q=1 h_q=128 S=4096, paged with 64-token blocks."""
    return make_workload("dense_paged_b32_h128_s4096", 32, 1, 128, [4096] * 32, 64, seed)


def config_sparse(seed: int = 1003) -> Workload:
    """DSA/SFA sparse: B=32 Q=1 h_q=128 S=32768 top_k=2048; 3 rows keep 1500 entries."""
    B = 32
    return make_workload("sparse_b32_h128_s32768_top2048", B, 1, 128, [32768] * B, 64, seed,
                         top_k=2048, short_rows=round(0.1 * B), short_valid=1500)


def config_split_kv(seed: int = 1004) -> Workload:
    """Split-KV: B=8 Q=1 h_q=128 S=131072, 8 shards interleaved by 64 tokens."""
    return make_workload("splitkv_b8_h128_s131072_n8_i64", 8, 1, 128, [131072] * 8, 64, seed,
                         num_shards=8, interleave=64)


def config_mtp(seed: int = 1005) -> Workload:
    """MTP sparse: B=128 Q=2 h_q=64, S log-uniform in [1024, 65536], top_k=min(2048,S),
    shared index list across the two query tokens, 1% of rows with x8 RoPE columns."""
    B = 128
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    S = np.rint(np.exp(g.uniform(math.log(1024.0), math.log(65536.0), size=B))).astype(np.int32)
    return make_workload("mtp_sparse_b128_q2_h64_top2048", B, 2, 64, S, 64, seed, top_k=2048,
                         outlier_rate=0.01, outlier_factor=8.0)


def config_dense_32k(seed: int = 1006) -> Workload:
    """Dense counterpart of the sparse config: B=32 Q=1 h_q=128 S=32768."""
    return make_workload("dense_paged_b32_h128_s32768", 32, 1, 128, [32768] * 32, 64, seed)


def config_sparse_dcp(seed: int = 1007) -> Workload:
    """Sparse top-k under DCP: the split-KV shape (B=8 Q=1 h_q=128 S=131072, 8
    shards interleaved by 64 tokens) attending a top_k=2048 list per sequence."""
    return make_workload("sparse_dcp_b8_h128_s131072_top2048_n8_i64", 8, 1, 128, [131072] * 8, 64, seed,
                         top_k=2048, num_shards=8, interleave=64)


PRESETS = {
    1: config_tiny,
    2: config_dense_paged,
    3: config_sparse,
    4: config_split_kv,
    5: config_mtp,
    6: config_dense_32k,
    7: config_sparse_dcp,
}


def rotate_indices(w: Workload, seed: int) -> np.ndarray:
    """A fresh index set with the same shape/statistics (used to defeat caches when timing)."""
    assert w.indices is not None
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 11])))
    lists = make_topk_indices(g, w.seq_lens, w.top_k, int(w.meta.get("short_rows", 0)),
                              int(w.meta.get("short_valid", 0)))
    if w.index_stride_q == 0:
        return lists
    return np.ascontiguousarray(np.repeat(lists[:, None, :], w.Q, axis=1))


def attended_count(w: Workload) -> int:
    """sum over (b, q) of |A(b,q)|: the positions each query token attends.

    Pure bookkeeping on integers (no attention arithmetic): dense counts causal
    positions (per shard summed over shards = the unsharded count); sparse counts
    valid list entries not beyond the causal limit.
    """
    total = 0
    for b in range(w.B):
        S = int(w.seq_lens[b])
        for qi in range(w.Q):
            last = S - w.Q + qi
            if w.indices is None:
                total += max(0, last + 1)
            else:
                lst = w.indices.reshape(-1)[b * w.index_stride_b + qi * w.index_stride_q:
                                            b * w.index_stride_b + qi * w.index_stride_q + w.top_k]
                total += int(np.count_nonzero((lst >= 0) & (lst <= last)))
    return total


@dataclass
class KvWriteInputs:
    """Seeded inputs of one latent-cache write: T new rows, their slots and positions."""
    rows: np.ndarray       # uint16 [T, 576] bf16 bits
    slots: np.ndarray      # int32 [T]: distinct slots, some -1 (not stored) and some >= num_slots
    positions: np.ndarray  # int32 [T]
    num_slots: int


def make_kv_write_inputs(T: int, num_slots: int, seed: int, skip_frac: float = 0.1,
                         out_of_range: int = 2, block_size: int = 64, seq_tokens: int = 4096) -> KvWriteInputs:
    """A prefill batch's new rows and their slot map, shaped like a paged cache's:
    the T tokens form sequences of up to `seq_tokens` tokens at positions 0, 1, ...;
    each sequence's blocks are distinct physical blocks drawn by a seeded
    permutation of the cache's num_slots / block_size blocks, and token p of a
    sequence goes to slot block[p / block_size] * block_size + p mod block_size
    (the DCP page's table A: slot_mapping into [N_blk, block_size, D]).  Rows are
    N(0,1) -> bf16 bits.  A skip_frac share of the slots is replaced by -1 and
    `out_of_range` entries by slots at or past the end of the cache.  Caches too
    small for whole blocks get distinct single slots."""
    g_rows, g_slots, _ = _children(seed, 3)
    rows = _normal_bf16(g_rows, (T, D_QK))
    lens = [min(seq_tokens, T - o) for o in range(0, T, seq_tokens)]
    bs = block_size
    if sum((n + bs - 1) // bs for n in lens) > num_slots // bs:
        bs = 1
    blocks = g_slots.permutation(num_slots // bs) if num_slots >= bs else np.zeros(0, dtype=np.int64)
    slots = np.empty(T, dtype=np.int32)
    positions = np.empty(T, dtype=np.int32)
    o = used = 0
    for n in lens:
        p = np.arange(n)
        nb = (n + bs - 1) // bs
        own = blocks[used:used + nb]
        used += nb
        if len(own) == nb:
            slots[o:o + n] = own[p // bs] * bs + p % bs
        else:  # more tokens than slots: wrap around the cache
            slots[o:o + n] = (o + p) % num_slots
        positions[o:o + n] = p
        o += n
    if T:
        skip = g_slots.random(T) < skip_frac
        slots[skip] = -1
        k = min(out_of_range, T)
        far = g_slots.choice(T, size=k, replace=False)
        slots[far] = num_slots + np.arange(k, dtype=np.int32)
    return KvWriteInputs(rows=rows, slots=slots, positions=positions, num_slots=num_slots)


@dataclass
class TopkInputs:
    """Seeded indexer scores for the top-k selection: float32 [B, Q, max_len]."""
    scores: np.ndarray
    seq_lens: np.ndarray   # int32 [B]
    top_k: int


def make_topk_scores(B: int, Q: int, seq_lens, top_k: int, seed: int, zero_frac: float = 0.25,
                     max_len: int = 0) -> TopkInputs:
    """N(0,1) scores rounded to bf16 precision (so equal scores occur, as from bf16
    indexer arithmetic), a `zero_frac` share set to exactly 0 (a ReLU-weighted
    score's zeros: long runs of ties), and +inf past each row's causal length
    S_b - Q + q + 1, so that a read beyond the row would be selected and seen."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    assert seq_lens.shape == (B,)
    max_len = max_len or int(seq_lens.max(initial=1))
    g_val, g_zero = _children(seed, 2)
    x = g_val.standard_normal((B, Q, max_len), dtype=np.float32)
    s = bf16_bits_to_f32(f32_to_bf16_bits(x)).reshape(B, Q, max_len)
    s[g_zero.random((B, Q, max_len)) < zero_frac] = 0.0
    for b in range(B):
        for q in range(Q):
            L = min(max(int(seq_lens[b]) - Q + q + 1, 0), max_len)
            s[b, q, L:] = np.inf
    return TopkInputs(scores=np.ascontiguousarray(s, dtype=np.float32), seq_lens=seq_lens, top_k=top_k)
