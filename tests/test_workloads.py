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


def test_generated_workloads_pass_the_device_data_validator():
    # the workload generators at reduced sizes (the same code paths as the
    # full-size presets: dense paging, short sparse rows, a list shared by Q = 2)
    from helpers import validate_device_inputs
    cases = [W.config_tiny(),
             W.make_workload("dense", 4, 1, 16, [4096, 77, 1, 300], 64, seed=1),
             W.make_workload("sparse", 10, 1, 16, [8192] * 10, 64, seed=2, top_k=2048, short_rows=3,
                             short_valid=1500),
             W.make_workload("mtp", 6, 2, 16, [1024, 1500, 3000, 5000, 2048, 4097], 64, seed=3, top_k=2048)]
    for w in cases:
        rep = validate_device_inputs(w)
        assert not rep["bad_seq_lens"] and not rep["bad_blocks"], w.name
        assert rep["out_of_range"] == 0 and rep["duplicates"] == 0, w.name
    assert validate_device_inputs(cases[2])["padding"] == 3 * (2048 - 1500)
    assert validate_device_inputs(cases[3])["padding"] == 2 * (2048 - 1024) + 2 * (2048 - 1500)


def test_validator_flags_what_the_device_would_skip():
    from helpers import validate_device_inputs
    w = W.make_workload("bad", 3, 2, 16, [100, 300, 64], 64, seed=5, top_k=40, shared_q_indices=False)
    w.block_table[1, 2] = w.kv.shape[0]         # block 2 of sequence 1 (positions 128..191) out of range
    w.block_table[0, 3] = -1                     # beyond S_0 = 100 (blocks 0, 1): never attended, not flagged
    w.seq_lens[2] = 1                            # below Q = 2
    idx = w.indices.reshape(3, 2, 40)
    masked0 = validate_device_inputs(w)["causal_masked"]
    idx[0, 0, :3] = [98, -5, 1000]               # 98 = pos(0, 0); -5 and 1000 are out of range
    idx[0, 1, 0] = idx[0, 1, 1]                  # a duplicate
    idx[0, 1, 2] = 99                            # pos(0, 1) = 99: in range
    idx[0, 0, 5] = 99                            # past pos(0, 0): masked for q = 0 only
    rep = validate_device_inputs(w)
    assert rep["bad_blocks"] == [(1, 2)] and rep["bad_seq_lens"] == [2]
    assert rep["out_of_range"] == 2 and rep["duplicates"] >= 1
    assert rep["causal_masked"] >= 1 and masked0 >= 0
