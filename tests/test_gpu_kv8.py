"""GPU parity of the int8 latent cache: the HIP path through the C ABI against
the fp64 oracle, which reads the same int8 codes and per-row factors (value =
factor x code).

Bars as for the bf16 cache (tests/parity.py: lse |Δ| <= 1e-3; O |Δ| <= 1e-2,
and for bf16 outputs 1 bf16 ulp where |O_ref| >= 4).  The kernel widens the
codes exactly (as code + 128 in bf16) and removes the bias in fp32, so the only
roundings beyond the bf16 cache's are fp32 ones and the bf16 rounding of the
factor-carrying P.V weights (relative 2^-9 per weight, averaging out over the
attended tokens).  The full-size workload over the int8 cache is compared on
every row in test_gpu_full_size.py.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
from latent_decode_attention_amd import mla_decode as md  # noqa: E402
from latent_decode_attention_amd import workloads as W  # noqa: E402
from latent_decode_attention_amd.device import upload, run  # noqa: E402
from test_gpu_parity import EDGE_SHAPES, assert_lse_close, assert_o_close  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def planner_shape():
    md.GROUP_ROWS = 0  # int8 caches always run with 64-row work-groups
    yield
    md.GROUP_ROWS = 0


def kv8(name, B, Q, h_q, S, bs, seed, **kw):
    return W.int8_cache(W.make_workload(name, B, Q, h_q, S, bs, seed, **kw))


CASES = {
    "dense_tiny": lambda: W.int8_cache(W.config_tiny()),
    "dense_ragged_h128": lambda: kv8("d128", 3, 1, 128, [700, 64, 1], 16, 11),
    "dense_q2_h64_split": lambda: kv8("dq2", 2, 2, 64, [300, 5000], 64, 12),
    "dense_q3_h32": lambda: kv8("dq3", 2, 3, 32, [3, 190], 32, 13),
    "sparse_shared": lambda: kv8("sps", 3, 2, 64, [900, 2000, 130], 64, 14, top_k=256),
    "sparse_per_token": lambda: kv8("spt", 2, 2, 128, [3000, 70], 64, 15, top_k=300, shared_q_indices=False),
    "sparse_short_rows": lambda: kv8("spr", 4, 1, 128, [4096] * 4, 64, 16, top_k=1024, short_rows=2,
                                     short_valid=100),
    "sparse_rope_outliers": lambda: kv8("spo", 2, 2, 64, [2500, 800], 64, 17, top_k=512,
                                        outlier_rate=0.05, outlier_factor=8.0),
}


def oracle_of(w, rows=None):
    return oracle.sparse(w, rows=rows) if w.indices is not None else oracle.dense(w, rows=rows)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_int8_cache_matches_the_oracle(name, out_dtype):
    w = CASES[name]()
    out, lse = run(upload(w), out_dtype=out_dtype)
    torch.cuda.synchronize()
    ro, rl = oracle_of(w)
    assert_o_close(out, ro, w.name)
    assert_lse_close(lse, rl, w.name)


@pytest.mark.parametrize("name", sorted(EDGE_SHAPES))
def test_int8_edge_shapes(name):
    """The limits of the supported range (1, 3 and 96 heads, 16 query tokens, 1-
    and 4096-token pages, a 65536-entry list, 600 sequences) over the int8 cache."""
    B, Q, h, lens, bs, k, shared = EDGE_SHAPES[name]
    w = W.int8_cache(W.make_workload(name, B, Q, h, lens, bs, seed=sum(map(ord, name)) + 1, top_k=k,
                                     shared_q_indices=shared, spare_blocks=2))
    out, lse = run(upload(w), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle_of(w)
    assert_o_close(out, ro, w.name)
    assert_lse_close(lse, rl, w.name)


def test_int8_cache_with_factors_over_a_wide_range():
    # Per-row factors log-uniform over 2^-10 .. 2^-2, codes re-derived from the
    # same unit-scale values (so coarse codes on some rows, clipped ones on
    # others), and 2% of the rows all zero with factor 0: the bias removal and
    # the factor-carrying weights must hold at every scale.  (The tolerances
    # assume values of unit scale, as everywhere else.)
    w = kv8("wide", 2, 1, 128, [1500, 333], 64, 18, top_k=0)
    g = np.random.default_rng(18)
    x = W.bf16_bits_to_f32(w.kv)
    poisoned = np.isnan(w.kv_scale)
    fac = (2.0 ** g.uniform(-10, -2, size=w.kv_scale.shape)).astype(np.float32)
    codes = np.clip(np.rint(np.nan_to_num(x) / fac[..., None]), -128, 127).astype(np.int8)
    zero = g.random(fac.shape) < 0.02
    codes[zero] = 0
    fac[zero] = 0.0
    w.kv8[:] = codes
    w.kv_scale[:] = np.where(poisoned, np.float32(np.nan), fac)
    out, lse = run(upload(w), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle_of(w)
    assert_o_close(out, ro, w.name)
    assert_lse_close(lse, rl, w.name)


def test_int8_extreme_codes():
    # Every code -128 or 127: the widened values 0 and 255 are the ends of the
    # exact range, and the bias removal cancels the largest sums.
    w = kv8("ext", 2, 2, 64, [640, 130], 64, 19, top_k=0)
    g = np.random.default_rng(19)
    w.kv8[:] = np.where(g.random(w.kv8.shape) < 0.5, -128, 127).astype(np.int8)
    out, lse = run(upload(w), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle_of(w)
    assert_o_close(out, ro, w.name)
    assert_lse_close(lse, rl, w.name)


@pytest.mark.parametrize("sparse", [False, True], ids=["dense", "sparse"])
def test_int8_dcp_shards_match_the_oracle(sparse):
    w = kv8("dcp", 2, 1, 128, [3000, 1100], 64, 20, top_k=512 if sparse else 0, num_shards=4, interleave=16)
    parts, lses = run(upload(w))
    merged, mlse = md.mla_merge_lse(parts, lses, out_dtype=torch.float32)
    torch.cuda.synchronize()
    f = oracle.sparse if sparse else oracle.dense
    for r in range(4):
        ro, rl = f(w, num_shards=4, interleave=16, shard_id=r)
        assert_o_close(parts[r], ro, f"shard {r}")
        assert_lse_close(lses[r], rl, f"shard {r}")
    ro, rl = f(w)
    assert_o_close(merged, ro, "merged")
    assert_lse_close(mlse, rl, "merged")


def test_int8_poisoned_factors_of_unreferenced_rows_never_reach_the_output():
    # Spare blocks carry NaN factors (the generator's poison) and the unused
    # block-table slots point at one of them; every attended row is finite.
    w = kv8("poison", 3, 1, 128, [257, 64, 1000], 64, 21, top_k=0, spare_blocks=4)
    assert np.isnan(w.kv_scale).any()
    out, lse = run(upload(w), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    ro, rl = oracle_of(w)
    assert_o_close(out, ro, w.name)


def test_int8_repeated_runs_are_bitwise_identical():
    w = CASES["sparse_shared"]()
    d = upload(w)
    a = run(d)
    b = run(d)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
