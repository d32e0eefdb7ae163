"""The top-k selection reference (oracle/topk.py) pinned to what its definition
fixes, independently of how it is computed: exhaustive search over every subset
on tiny rows, an independent library route (argpartition) for distinct scores,
and the special cases (short rows, all-equal scores, NaN, signed zeros, causal
row lengths).  Planted mistakes in a copy of the reference must fail a pin."""
import itertools
import types

import numpy as np
import pytest

from oracle import topk
from latent_decode_attention_amd import workloads as W

VALUES = [-np.inf, -1.0, -0.0, 0.0, 0.5, 1.0, np.inf, np.nan]


def beats(s, i, j):
    """Position i ranks above position j: numbers above NaN, larger above smaller,
    equal (or both NaN) by lower position."""
    ni, nj = np.isnan(s[i]), np.isnan(s[j])
    if ni != nj:
        return nj
    if not ni and s[i] != s[j]:
        return s[i] > s[j]
    return i < j


def test_exhaustive_search_on_tiny_rows():
    g = np.random.default_rng(3)
    for trial in range(400):
        L = int(g.integers(0, 8))
        k = int(g.integers(1, 9))
        s = np.array(g.choice(VALUES, size=L), dtype=np.float32)
        m = min(k, L)
        winners = [set(c) for c in itertools.combinations(range(L), m)
                   if all(beats(s, i, j) for i in c for j in range(L) if j not in c)]
        assert len(winners) == 1, (s, k)
        want = sorted(winners[0]) + [-1] * (k - m)
        assert topk.select_row(s, k).tolist() == want, (s, k)


@pytest.mark.parametrize("L,k", [(1000, 1), (1000, 37), (4096, 2048), (2049, 2048)])
def test_distinct_scores_agree_with_argpartition(L, k):
    g = np.random.default_rng(L + k)
    s = g.permutation(L).astype(np.float32) * np.float32(0.25) - np.float32(100.0)  # distinct, exact
    got = topk.select_row(s, k)
    assert set(got.tolist()) == set(np.argpartition(-s.astype(np.float64), k - 1)[:k].tolist())
    assert np.all(np.diff(got) > 0) and got.dtype == np.int32


def test_short_rows_take_every_position_then_pad():
    s = np.array([3.0, -1.0, np.nan, 0.0, 7.0], dtype=np.float32)
    assert topk.select_row(s, 8).tolist() == [0, 1, 2, 3, 4, -1, -1, -1]
    assert topk.select_row(s[:0], 3).tolist() == [-1, -1, -1]


def test_equal_scores_take_the_lowest_positions():
    assert topk.select_row(np.zeros(50, dtype=np.float32), 7).tolist() == list(range(7))
    s = np.full(20, 2.0, dtype=np.float32)
    s[[3, 11]] = 5.0
    assert topk.select_row(s, 4).tolist() == [0, 1, 3, 11]


def test_nan_ranks_below_every_number():
    s = np.array([np.nan, -np.inf, np.nan, -5.0], dtype=np.float32)
    assert topk.select_row(s, 2).tolist() == [1, 3]
    assert topk.select_row(s, 3).tolist() == [0, 1, 3]


def test_signed_zeros_are_equal():
    assert topk.select_row(np.array([-0.0, 0.0], dtype=np.float32), 1).tolist() == [0]
    assert topk.select_row(np.array([0.0, -0.0], dtype=np.float32), 1).tolist() == [0]


def test_rows_stop_at_the_causal_limit():
    # Q = 3 query tokens of a sequence of length 10: token q selects among
    # positions 0 .. 7 + q.  Past the limit the scores are +inf (never selected);
    # the last allowed position carries the row's largest finite score.
    x = W.make_topk_scores(2, 3, [10, 4], 5, seed=8)
    for b, S in enumerate((10, 4)):
        for q in range(3):
            last = S - 3 + q
            if last >= 0:
                x.scores[b, q, last] = 1e30
    got = topk.select(x.scores, x.seq_lens, 5)
    for b, S in enumerate((10, 4)):
        for q in range(3):
            L = S - 3 + q + 1
            row = got[b, q]
            assert np.all(row[row >= 0] < L) and (row >= 0).sum() == min(5, L)
            assert L - 1 in row.tolist()


def test_generator_puts_infinity_past_each_row():
    x = W.make_topk_scores(3, 2, [5, 1, 9], 4, seed=2, max_len=12)
    for b, S in enumerate((5, 1, 9)):
        for q in range(2):
            L = max(S - 2 + q + 1, 0)
            assert np.all(np.isposinf(x.scores[b, q, L:])) and np.all(np.isfinite(x.scores[b, q, :L]))


# ------------------------------------------------------------------ planted mistakes

MUTATIONS = {
    "ties_by_higher_position": ("np.lexsort((pos, -value, is_nan))", "np.lexsort((-pos, -value, is_nan))"),
    "nan_ranks_first": ("np.lexsort((pos, -value, is_nan))", "np.lexsort((pos, -value, ~is_nan))"),
    "smallest_instead_of_largest": ("np.lexsort((pos, -value, is_nan))", "np.lexsort((pos, value, is_nan))"),
    "causal_limit_off_by_one": ("seq_len - Q + q + 1", "seq_len - Q + q"),
    "result_in_rank_order": ("chosen = np.sort(ranked[:min(top_k, L)])", "chosen = ranked[:min(top_k, L)]"),
    "padding_with_zero": ("out = np.full(top_k, -1, dtype=np.int32)", "out = np.zeros(top_k, dtype=np.int32)"),
    "one_too_few": ("ranked[:min(top_k, L)]", "ranked[:min(top_k, L) - 1]"),
}

PINS = [test_exhaustive_search_on_tiny_rows, test_short_rows_take_every_position_then_pad,
        test_equal_scores_take_the_lowest_positions, test_nan_ranks_below_every_number,
        test_signed_zeros_are_equal, test_rows_stop_at_the_causal_limit,
        lambda: test_distinct_scores_agree_with_argpartition(1000, 37)]


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, monkeypatch):
    src = open(topk.__file__).read()
    old, new = MUTATIONS[mutation]
    assert src.count(old) >= 1, "mutation anchor must exist"
    mod = types.ModuleType("mutated_topk")
    exec(compile(src.replace(old, new), "mutated_topk.py", "exec"), mod.__dict__)
    for name in ("row_length", "select_row", "select"):
        monkeypatch.setattr(topk, name, getattr(mod, name))
    caught = 0
    for pin in PINS:
        try:
            pin()
        except Exception:  # an assertion or a crash both count as caught
            caught += 1
    assert caught, "no pin detects mutation %s" % mutation
