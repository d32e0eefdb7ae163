"""The latent-cache write reference (oracle/cache_ops.py) against what the DCP
page's table A fixes ("RFC: MsModeling 支持 Decode Context Parallel 仿真",
§2.1.4.1): rows land at their slots and nowhere else, skipped tokens change
nothing, the shards of an interleaved DCP group partition the tokens, and a row
written at slot row(b, p) is the row the attention reads for position p."""
import numpy as np
import pytest

import oracle
from oracle import cache_ops
from latent_decode_attention_amd import workloads as W


def _cache(num_slots, seed):
    g = np.random.default_rng(seed)
    return g.integers(0, 1 << 16, size=(num_slots, W.D_QK), dtype=np.uint16)


@pytest.mark.parametrize("T,num_slots", [(0, 10), (1, 5), (37, 100), (500, 4096)])
def test_rows_land_at_their_slots_and_nowhere_else(T, num_slots):
    x = W.make_kv_write_inputs(T, num_slots, seed=T + num_slots)
    kv = _cache(num_slots, 3)
    got = cache_ops.kv_write(kv, x.rows, x.slots)
    stored = (x.slots >= 0) & (x.slots < num_slots)
    assert np.array_equal(got[x.slots[stored]], x.rows[stored])
    untouched = np.ones(num_slots, dtype=bool)
    untouched[x.slots[stored]] = False
    assert np.array_equal(got[untouched], kv[untouched])
    assert not np.shares_memory(got, kv)


def test_skipped_tokens_change_nothing():
    x = W.make_kv_write_inputs(64, 256, seed=5)
    kv = _cache(256, 4)
    none = np.full_like(x.slots, -1)
    assert np.array_equal(cache_ops.kv_write(kv, x.rows, none), kv)
    far = np.arange(64, dtype=np.int32) + 256
    assert np.array_equal(cache_ops.kv_write(kv, x.rows, far), kv)


def test_token_order_does_not_matter_for_distinct_slots():
    x = W.make_kv_write_inputs(300, 1000, seed=6)
    kv = _cache(1000, 7)
    perm = np.random.default_rng(8).permutation(300)
    assert np.array_equal(cache_ops.kv_write(kv, x.rows, x.slots),
                          cache_ops.kv_write(kv, x.rows[perm], x.slots[perm]))


@pytest.mark.parametrize("N,I", [(2, 1), (8, 64), (3, 7)])
def test_interleaved_shards_partition_the_tokens(N, I):
    x = W.make_kv_write_inputs(700, 2000, seed=N * 10 + I)
    kv = _cache(2000, 9)
    whole = cache_ops.kv_write(kv, x.rows, x.slots)
    step = kv
    for r in range(N):
        step = cache_ops.kv_write(step, x.rows, x.slots, x.positions, N, I, r)
    assert np.array_equal(step, whole)
    # each shard alone stores exactly the tokens it owns
    owners = cache_ops.shard_of(x.positions, N, I)
    for r in range(N):
        mine = cache_ops.kv_write(kv, x.rows, x.slots, x.positions, N, I, r)
        sl = x.slots.copy()
        sl[owners != r] = -1
        assert np.array_equal(mine, cache_ops.kv_write(kv, x.rows, sl))


def test_written_rows_are_the_rows_attention_reads():
    # Overwrite the last 40 positions of each sequence with garbage, then store the
    # original rows back through slots row(b, p) = block_table[b, p / bs] * bs + p % bs:
    # the cache, and so the attention the oracle computes over it, is restored.
    w = W.make_workload("kvw", 2, 1, 16, [300, 170], 16, seed=21)
    bs = w.block_size
    flat = w.kv.reshape(-1, W.D_QK)
    rows, slots = [], []
    for b, S in enumerate(w.seq_lens):
        for p in range(S - 40, S):
            slot = int(w.block_table[b, p // bs]) * bs + p % bs
            rows.append(flat[slot].copy())
            slots.append(slot)
    rows, slots = np.stack(rows), np.array(slots, dtype=np.int32)
    damaged = flat.copy()
    damaged[slots] = 0x7FC0  # bf16 NaN
    restored = cache_ops.kv_write(damaged, rows, slots)
    assert np.array_equal(restored, flat)
    o_ref, l_ref = oracle.dense(w)
    w.kv = restored.reshape(w.kv.shape)
    o_new, l_new = oracle.dense(w)
    assert np.array_equal(o_new, o_ref) and np.array_equal(l_new, l_ref)
