"""Pins of the fp64 oracle to things other than itself.

Each test fixes the oracle against a library routine (scipy's softmax and
logsumexp on the logical, unpaged rows), a closed form, a hand-derived golden
fixture or an invariant the pages state (shards + online-softmax merge equal the
unsharded result: "RFC: MsModeling 支持 Decode Context Parallel 仿真" §1.1 and
§2.1.4.3; sparse attention is the dense formula over the selected positions:
same page §1.3).  Together they are meant to catch a dropped term, a wrong
sign, a wrong index, a transposed operand or a wrong attended set.
"""
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
from helpers import bf16, f64, paged, random_rows, workload
from latent_decode_attention_amd.workloads import D_QK, D_V, Workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _library_route(q_bits, logical, scale, A_of):
    """softmax / logsumexp (scipy) on logical rows; A_of(b, q) gives the attended positions."""
    B, Q, H, _ = q_bits.shape
    out = np.zeros((B, Q, H, D_V))
    lse = np.full((B, Q, H), -np.inf)
    for b in range(B):
        K = f64(logical[b])                       # [S, 576]
        for qi in range(Q):
            A = np.asarray(A_of(b, qi), dtype=np.int64)
            if A.size == 0:
                continue
            for h in range(H):
                s = scale * (K[A] @ f64(q_bits[b, qi, h]))
                lse[b, qi, h] = logsumexp(s)
                out[b, qi, h] = softmax(s) @ K[A, :D_V]
    return out.reshape(-1, D_V), lse.reshape(-1)


def test_dense_matches_library_route_paged_ragged_causal():
    rng = np.random.default_rng(1)
    S = [37, 70, 5]
    Q, H = 2, 3
    logical = [random_rows(rng, s) for s in S]
    q = random_rows(rng, len(S) * Q * H).reshape(len(S), Q, H, D_QK)
    w = workload(q, logical, block_size=16, seed=2)
    out, lse = oracle.dense(w)
    ref_o, ref_l = _library_route(q, logical, w.scale, lambda b, qi: np.arange(S[b] - Q + qi + 1))
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-12)


def test_sparse_matches_library_route_with_padding_and_out_of_range():
    rng = np.random.default_rng(3)
    S = [50, 90]
    Q, H, top_k = 2, 2, 12
    logical = [random_rows(rng, s) for s in S]
    q = random_rows(rng, len(S) * Q * H).reshape(len(S), Q, H, D_QK)
    idx = np.full((len(S), Q, top_k), -1, dtype=np.int32)
    idx[0, 0, :6] = [3, 49, 7, 48, 0, 20]      # 49 is beyond q=0's causal limit (48)
    idx[0, 1, :7] = [3, 49, 7, 48, 0, 20, 200]  # 200 is out of range
    idx[1, 0, :12] = rng.choice(89, 12, replace=False)
    idx[1, 1, :3] = [89, 1, 1]                 # duplicate counts twice
    w = workload(q, logical, block_size=8, seed=4, indices=idx.reshape(-1), top_k=top_k,
                 index_stride_b=Q * top_k, index_stride_q=top_k)
    out, lse = oracle.sparse(w)

    def A_of(b, qi):
        last = S[b] - Q + qi
        return [i for i in idx[b, qi] if 0 <= i <= last]

    ref_o, ref_l = _library_route(q, logical, w.scale, A_of)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-12)


def test_scale_zero_gives_mean_of_v_and_log_count():
    rng = np.random.default_rng(5)
    S = [33, 64]
    logical = [random_rows(rng, s) for s in S]
    q = random_rows(rng, 2 * 1 * 4).reshape(2, 1, 4, D_QK)
    w = workload(q, logical, block_size=32, scale=0.0, seed=6)
    out, lse = oracle.dense(w)
    for b in range(2):
        mean = f64(logical[b])[:, :D_V].mean(axis=0)
        for h in range(4):
            np.testing.assert_allclose(out[b * 4 + h], mean, atol=1e-13)
            assert abs(lse[b * 4 + h] - math.log(S[b])) < 1e-13


def test_identical_keys_give_mean_of_v_plus_constant_lse():
    # Scores use only the RoPE columns (q[:512] = 0) and every row carries the
    # same RoPE part, so all scores equal c = scale * <q_rope, k_rope>.
    rng = np.random.default_rng(7)
    S = 40
    rows = random_rows(rng, S)
    rope = bf16(rng.integers(-3, 4, size=64).astype(np.float32))
    rows[:, 512:] = rope
    q = np.zeros((1, 1, 2, D_QK), dtype=np.uint16)
    q[0, 0, :, 512:] = bf16(rng.integers(-2, 3, size=(2, 64)).astype(np.float32))
    w = workload(q, [rows], block_size=16, seed=8)
    out, lse = oracle.dense(w)
    for h in range(2):
        c = w.scale * float(np.dot(f64(q[0, 0, h, 512:]), f64(rope)))
        np.testing.assert_allclose(out[h], f64(rows)[:, :D_V].mean(axis=0), atol=1e-13)
        assert abs(lse[h] - (c + math.log(S))) < 1e-12


@pytest.mark.parametrize("score_cols", ["rope", "nope"])
def test_two_tokens_logistic_closed_form(score_cols):
    # A = {0, 1}: weights are the logistic function of s0 - s1, lse = logaddexp.
    rng = np.random.default_rng(9)
    rows = bf16(rng.integers(-4, 5, size=(2, D_QK)).astype(np.float32))
    q = np.zeros((1, 1, 1, D_QK), dtype=np.uint16)
    cols = slice(512, 576) if score_cols == "rope" else slice(0, 512)
    q[0, 0, 0, cols] = bf16(rng.integers(-1, 2, size=cols.stop - cols.start).astype(np.float32))
    scale = 1.0 / 16
    w = workload(q, [rows], block_size=16, scale=scale, seed=10)
    out, lse = oracle.dense(w)
    qq = f64(q[0, 0, 0])
    s0, s1 = scale * np.dot(qq, f64(rows[0])), scale * np.dot(qq, f64(rows[1]))
    sig = 1.0 / (1.0 + math.exp(s1 - s0))
    expect = sig * f64(rows[0])[:D_V] + (1 - sig) * f64(rows[1])[:D_V]
    np.testing.assert_allclose(out[0], expect, atol=1e-13)
    assert abs(lse[0] - np.logaddexp(s0, s1)) < 1e-13


def test_single_token_gives_v_and_its_score():
    rng = np.random.default_rng(11)
    rows = random_rows(rng, 1)
    q = random_rows(rng, 3).reshape(1, 1, 3, D_QK)
    w = workload(q, [rows], block_size=16, seed=12)
    out, lse = oracle.dense(w)
    for h in range(3):
        np.testing.assert_array_equal(out[h], f64(rows[0])[:D_V])
        s = w.scale * float(np.dot(f64(q[0, 0, h]), f64(rows[0])))
        assert abs(lse[h] - s) < 1e-12


def _one_hot_rows(S):
    """K part zero (all scores 0), V row p = one-hot(p): O[c] = [c in A] / |A|."""
    assert S <= D_V
    rows = np.zeros((S, D_QK), dtype=np.uint16)
    rows[np.arange(S), np.arange(S)] = bf16(1.0)
    return rows


def _attended_from_probe(out_row, lse_val):
    n = int(round(math.exp(lse_val))) if np.isfinite(lse_val) else 0
    got = {int(c) for c in np.nonzero(out_row > 0)[0]}
    return n, got


def test_one_hot_probe_recovers_causal_and_sharded_sets():
    S, Q = 45, 2
    rows = _one_hot_rows(S)
    q = np.zeros((1, Q, 1, D_QK), dtype=np.uint16)   # every score is 0
    w = workload(q, [rows], block_size=8, seed=14)
    for N, I in [(1, 1), (3, 2), (4, 8), (8, 64)]:
        for r in range(N):
            out, lse = oracle.dense(w, num_shards=N, interleave=I, shard_id=r)
            for qi in range(Q):
                A = {p for p in range(S - Q + qi + 1) if (p // I) % N == r}
                n, got = _attended_from_probe(out[qi], lse[qi])
                assert got == A and n == len(A)
                if A:
                    np.testing.assert_allclose(out[qi][sorted(A)], 1.0 / len(A), atol=1e-15)


def test_one_hot_probe_sparse_multiplicity_and_padding():
    S = 30
    rows = _one_hot_rows(S)
    q = np.zeros((1, 1, 1, D_QK), dtype=np.uint16)
    idx = np.array([4, 4, -1, 29, 31, 0, -1, 17], dtype=np.int32)  # 4 twice; 31 out of range
    w = workload(q, [rows], block_size=4, seed=15, indices=idx, top_k=8, index_stride_b=8,
                 index_stride_q=0)
    out, lse = oracle.sparse(w)
    assert abs(lse[0] - math.log(5)) < 1e-14
    expect = np.zeros(D_V)
    expect[[0, 17, 29]] = 1 / 5
    expect[4] = 2 / 5
    np.testing.assert_allclose(out[0], expect, atol=1e-15)


@pytest.mark.parametrize("N,I", [(2, 1), (3, 4), (8, 2)])
def test_one_hot_probe_sparse_shards_keep_the_entries_each_shard_holds(N, I):
    S = 30
    rows = _one_hot_rows(S)
    q = np.zeros((1, 1, 1, D_QK), dtype=np.uint16)
    idx = np.array([4, 4, -1, 29, 31, 0, -1, 17, 9, 22, 13, 5], dtype=np.int32)
    w = workload(q, [rows], block_size=4, seed=15, indices=idx, top_k=12, index_stride_b=12,
                 index_stride_q=0)
    for r in range(N):
        out, lse = oracle.sparse(w, num_shards=N, interleave=I, shard_id=r)
        mine = [int(i) for i in idx if 0 <= i < S and (i // I) % N == r]
        if not mine:
            assert lse[0] == -np.inf and np.all(out[0] == 0)
            continue
        assert abs(lse[0] - math.log(len(mine))) < 1e-14
        expect = np.zeros(D_V)
        for i in mine:
            expect[i] += 1 / len(mine)
        np.testing.assert_allclose(out[0], expect, atol=1e-15)


@pytest.mark.parametrize("N,I", [(2, 1), (3, 4), (8, 16)])
def test_sparse_shards_then_merge_equal_unsharded(N, I):
    rng = np.random.default_rng(40 + N)
    S = [300, 129, 77]
    Q, H, K = 2, 2, 64
    logical = [random_rows(rng, s) for s in S]
    q = random_rows(rng, len(S) * Q * H).reshape(len(S), Q, H, D_QK)
    idx = np.full((len(S), Q, K), -1, dtype=np.int32)
    for b, s in enumerate(S):
        for qi in range(Q):
            n = min(K - 3, s)
            idx[b, qi, :n] = rng.choice(s, size=n, replace=False)
    w = workload(q, logical, block_size=16, seed=41, indices=idx.reshape(-1), top_k=K,
                 index_stride_b=Q * K, index_stride_q=K)
    full_o, full_l = oracle.sparse(w)
    parts = [oracle.sparse(w, num_shards=N, interleave=I, shard_id=r) for r in range(N)]
    mo, ml = oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(ml, full_l, rtol=0, atol=1e-12)
    np.testing.assert_allclose(mo, full_o, rtol=0, atol=1e-12)


def test_empty_attended_set_gives_zero_and_minus_inf():
    rng = np.random.default_rng(16)
    rows = random_rows(rng, 10)
    q = random_rows(rng, 2).reshape(1, 1, 2, D_QK)
    idx = np.full(6, -1, dtype=np.int32)
    w = workload(q, [rows], block_size=4, seed=17, indices=idx, top_k=6, index_stride_b=6)
    out, lse = oracle.sparse(w)
    assert np.all(out == 0) and np.all(lse == -np.inf)
    # a shard that owns no position of a short sequence
    out, lse = oracle.dense(w, num_shards=4, interleave=8, shard_id=3)
    assert np.all(out == 0) and np.all(lse == -np.inf)


def test_golden_three_token_fixture():
    """Hand-derived example stored in tests/golden (its derivation is in the file)."""
    vals = {}
    with open(os.path.join(GOLDEN, "three_token_closed_form.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=")
                vals[k.strip()] = float(v)
    rows = np.zeros((3, D_QK), dtype=np.uint16)
    rows[:, 512] = bf16([0.0, 1.0, 2.0])       # RoPE column 512 carries the score
    rows[0, 0] = bf16(1.0)                      # v0 = e0
    rows[1, 1] = bf16(2.0)                      # v1 = 2 e1
    rows[2, 0], rows[2, 2] = bf16(-1.0), bf16(1.0)  # v2 = -e0 + e2
    q = np.zeros((1, 1, 1, D_QK), dtype=np.uint16)
    q[0, 0, 0, 512] = bf16(16.0)
    w = workload(q, [rows], block_size=2, scale=1.0 / 16, seed=18)
    out, lse = oracle.dense(w)
    assert abs(lse[0] - vals["lse"]) < 1e-14
    for c in range(3):
        assert abs(out[0, c] - vals["O%d" % c]) < 1e-14
    assert np.all(out[0, 3:] == 0)


@pytest.mark.parametrize("N,I", [(1, 1), (2, 1), (3, 4), (8, 16)])
def test_shards_then_merge_equal_unsharded(N, I):
    rng = np.random.default_rng(19 + N)
    S = [129, 7, 300]
    Q, H = 2, 2
    logical = [random_rows(rng, s) for s in S]
    q = random_rows(rng, len(S) * Q * H).reshape(len(S), Q, H, D_QK)
    w = workload(q, logical, block_size=16, seed=20)
    full_o, full_l = oracle.dense(w)
    parts = [oracle.dense(w, num_shards=N, interleave=I, shard_id=r) for r in range(N)]
    mo, ml = oracle.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(ml, full_l, rtol=0, atol=1e-12)
    np.testing.assert_allclose(mo, full_o, rtol=0, atol=1e-12)


def test_sparse_over_all_positions_equals_dense_in_any_order():
    rng = np.random.default_rng(23)
    S = [60, 33]
    Q, H = 1, 3
    logical = [random_rows(rng, s) for s in S]
    q = random_rows(rng, len(S) * Q * H).reshape(len(S), Q, H, D_QK)
    top_k = 64
    idx = np.full((2, top_k), -1, dtype=np.int32)
    for b, s in enumerate(S):
        idx[b, :s] = rng.permutation(s)
    w = workload(q, logical, block_size=16, seed=24, indices=idx.reshape(-1), top_k=top_k,
                 index_stride_b=top_k, index_stride_q=0)
    d_o, d_l = oracle.dense(w)
    s_o, s_l = oracle.sparse(w)
    np.testing.assert_allclose(s_l, d_l, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s_o, d_o, rtol=0, atol=1e-12)


def test_padding_equals_shorter_list():
    rng = np.random.default_rng(25)
    logical = [random_rows(rng, 200)]
    q = random_rows(rng, 4).reshape(1, 1, 4, D_QK)
    sel = np.sort(rng.choice(200, 48, replace=False)).astype(np.int32)
    padded = np.concatenate([sel[:30], np.full(18, -1, np.int32)])
    w = workload(q, logical, block_size=16, seed=26)
    a = oracle.sparse(w, indices=padded, top_k=48, stride_b=48, stride_q=0)
    b = oracle.sparse(w, indices=sel[:30].copy(), top_k=30, stride_b=30, stride_q=0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_causal_first_token_equals_shorter_single_token_call():
    rng = np.random.default_rng(27)
    logical = [random_rows(rng, 77)]
    q2 = random_rows(rng, 2 * 3).reshape(1, 2, 3, D_QK)
    w2 = workload(q2, logical, block_size=16, seed=28)
    w1 = workload(np.ascontiguousarray(q2[:, :1]), [logical[0][:76]], block_size=16, seed=29)
    o2, l2 = oracle.dense(w2)
    o1, l1 = oracle.dense(w1)
    np.testing.assert_array_equal(o2[:3], o1)
    np.testing.assert_array_equal(l2[:3], l1)


def test_block_permutation_invariance():
    rng = np.random.default_rng(31)
    logical = [random_rows(rng, 150), random_rows(rng, 90)]
    q = random_rows(rng, 2 * 2).reshape(2, 1, 2, D_QK)
    a = oracle.dense(workload(q, logical, block_size=16, seed=32))
    b = oracle.dense(workload(q, logical, block_size=16, seed=33, spare=5))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_unused_poisoned_blocks_are_never_read():
    rng = np.random.default_rng(34)
    logical = [random_rows(rng, 20), random_rows(rng, 60)]
    q = random_rows(rng, 2).reshape(2, 1, 1, D_QK)
    w = workload(q, logical, block_size=16, seed=35, spare=3)
    # sequence 0 uses two blocks; its remaining table slots point at a NaN-filled spare
    assert w.block_table.shape[1] == 4
    assert np.isnan(f64(w.kv[w.block_table[0, 3]])).all()
    out, lse = oracle.dense(w)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_merge_identities():
    rng = np.random.default_rng(37)
    o = rng.standard_normal((3, 5, 7))
    l = rng.standard_normal((3, 5))
    # n = 1 is the identity
    mo, ml = oracle.merge(o[:1], l[:1])
    np.testing.assert_array_equal(mo, o[0])
    np.testing.assert_array_equal(ml, l[0])
    # a -inf part carries no weight
    l2 = np.stack([l[0], np.full(5, -np.inf)])
    o2 = np.stack([o[0], np.full((5, 7), 1e30)])
    mo, ml = oracle.merge(o2, l2)
    np.testing.assert_allclose(mo, o[0], atol=1e-15)
    np.testing.assert_allclose(ml, l[0], atol=1e-15)
    # equal outputs merge to that output; lse is logsumexp of the parts (scipy)
    same = np.repeat(o[:1], 3, axis=0)
    mo, ml = oracle.merge(same, l)
    np.testing.assert_allclose(mo, o[0], atol=1e-14)
    np.testing.assert_allclose(ml, logsumexp(l, axis=0), atol=1e-14)
    # all parts empty
    mo, ml = oracle.merge(o, np.full((3, 5), -np.inf))
    assert np.all(mo == 0) and np.all(ml == -np.inf)


def test_merge_weights_are_normalised_softmax_of_lse():
    rng = np.random.default_rng(38)
    o = rng.standard_normal((4, 6, 3))
    l = rng.standard_normal((4, 6)) * 5
    mo, ml = oracle.merge(o, l)
    w = softmax(l, axis=0)
    np.testing.assert_allclose(mo, np.einsum("nr,nrc->rc", w, o), atol=1e-13)
    np.testing.assert_allclose(ml, logsumexp(l, axis=0), atol=1e-13)


# ---- int8 latent cache.  The pages name a one-byte cache element but no
# dequantisation rule; the reading is value = (row factor) x (signed code).  Pin:
# codes times power-of-two factors are exact bf16 numbers, so the oracle over
# the int8 cache must give bit for bit what it gives over a bf16 cache holding
# those values (the bf16 reading being pinned by everything above).  Random
# per-row exponents catch a factor taken from the wrong row or dropped; codes
# spanning [-128, 127] catch an unsigned reading.

def _int8_pair(seed: int, per_row: bool, sparse: bool):
    from dataclasses import replace
    from latent_decode_attention_amd import workloads as W
    w = W.make_workload("kv8pin", 2, 2, 16, [37, 100], 16, seed, top_k=48 if sparse else 0,
                        shared_q_indices=False)
    g = np.random.default_rng(seed)
    codes = g.integers(-128, 128, size=w.kv.shape).astype(np.int8)
    if per_row:
        fac = (2.0 ** g.integers(-12, 3, size=w.kv.shape[:2])).astype(np.float32)
    else:
        fac = np.ones(w.kv.shape[:2], dtype=np.float32)
    vals = codes.astype(np.float64) * fac[..., None].astype(np.float64)
    kvb = bf16(vals.astype(np.float32))
    assert np.array_equal(f64(kvb), vals), "the values must be exact in bf16 for this pin"
    return replace(w, kv8=codes, kv_scale=fac), replace(w, kv=kvb)


@pytest.mark.parametrize("per_row,sparse", [(False, False), (True, False), (True, True)])
def test_int8_cache_equals_bf16_cache_of_the_same_values(per_row, sparse):
    w8, wb = _int8_pair(41 + per_row + 2 * sparse, per_row, sparse)
    run = oracle.sparse if sparse else oracle.dense
    o8, l8 = run(w8)
    ob, lb = run(wb)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)
    assert np.isfinite(o8).all()
