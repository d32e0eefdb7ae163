"""The seeded input module: determinism, bf16 rounding, block tables, index lists."""
import math

import numpy as np
import torch

from latent_decode_attention_amd import workloads as W


def test_bf16_rounding_matches_torch_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -2.5, 3.0039062, 1.00390625, 1.01171875, 0.0, -0.0], np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_same_seed_same_bytes_and_seed_changes_them():
    a = W.make_workload("t", 3, 2, 8, [100, 64, 5], 16, seed=5, top_k=32)
    b = W.make_workload("t", 3, 2, 8, [100, 64, 5], 16, seed=5, top_k=32)
    c = W.make_workload("t", 3, 2, 8, [100, 64, 5], 16, seed=6, top_k=32)
    for f in ("q", "kv", "block_table", "indices"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.kv, c.kv) and not np.array_equal(a.indices, c.indices)


def test_block_table_is_a_permutation_and_unused_slots_hit_poison():
    w = W.make_workload("t", 4, 1, 16, [100, 64, 5, 17], 16, seed=7, spare_blocks=3)
    nblk = [(s + 15) // 16 for s in w.seq_lens]
    used = np.concatenate([w.block_table[b, :n] for b, n in enumerate(nblk)])
    assert len(set(used.tolist())) == len(used) == sum(nblk)
    assert w.num_blocks == sum(nblk) + 3
    for b, n in enumerate(nblk):
        for j in range(n, w.max_blocks):
            assert np.isnan(W.bf16_bits_to_f32(w.kv[w.block_table[b, j]])).all()
    assert np.isfinite(W.bf16_bits_to_f32(w.kv[used])).all()


def test_topk_lists_sorted_distinct_in_range_with_short_rows():
    g = np.random.default_rng(1)
    S = [32768] * 32
    idx = W.make_topk_indices(g, S, 2048, short_rows=3, short_valid=1500)
    n_valid = (idx >= 0).sum(axis=1)
    assert sorted(n_valid.tolist()) == [1500] * 3 + [2048] * 29
    for b in range(32):
        v = idx[b][idx[b] >= 0]
        assert np.all(np.diff(v) > 0) and v.min() >= 0 and v.max() < 32768
        assert np.all(idx[b, n_valid[b]:] == -1)


def test_mtp_lengths_and_topk():
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([1005, 7])))
    S = np.rint(np.exp(g.uniform(math.log(1024.0), math.log(65536.0), size=128))).astype(np.int32)
    assert S.min() >= 1024 and S.max() <= 65536
    idx = W.make_topk_indices(np.random.default_rng(2), S, 2048)
    for b in range(128):
        assert (idx[b] >= 0).sum() == min(2048, S[b])


def test_outliers_scale_only_rope_columns():
    g1, g2, g3 = (np.random.default_rng(s) for s in (1, 2, 3))
    kv, _ = W.make_paged_cache(g1, g2, [640], 64, spare_blocks=0, outlier_rng=g3, outlier_rate=0.2)
    base, _ = W.make_paged_cache(np.random.default_rng(1), np.random.default_rng(2), [640], 64,
                                 spare_blocks=0)
    a, b = W.bf16_bits_to_f32(kv), W.bf16_bits_to_f32(base)
    np.testing.assert_array_equal(a[:, :, :512], b[:, :, :512])
    ratio = a[:, :, 512:] / np.where(b[:, :, 512:] == 0, 1, b[:, :, 512:])
    hit = np.all(np.isclose(ratio, 8.0) | (b[:, :, 512:] == 0), axis=-1)
    frac = hit.mean()
    assert 0.1 < frac < 0.3


def test_attended_count_bookkeeping():
    w = W.make_workload("t", 2, 2, 4, [10, 3], 4, seed=1)
    assert W.attended_count(w) == (9 + 10) + (2 + 3)
