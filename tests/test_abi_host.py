"""Host-only checks of the C ABI: the library loads, exports what the header
declares, rejects bad arguments before touching the device, and plans split-KV
partitions that cover every token exactly once."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")

md = pytest.importorskip("latent_decode_attention_amd.mla_decode",
                         reason="libmla_decode.so not built (run __graft_entry__.build())")
lib = md.lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("mla_decode_dense", "mla_decode_sparse", "mla_merge_lse", "mla_workspace_size",
                 "mla_status_string", "mla_plan_query"):
        assert want in names


def test_library_exports_every_declared_symbol():
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code, name in md.STATUS_NAMES.items():
        assert md.mla_status_string(code).startswith(name)
    assert "unknown" in md.mla_status_string(99)


FAKE = 0x10000  # never dereferenced: every case below fails validation first


def problem(**kw):
    base = dict(B=2, Q=1, h_q=128, d_qk=576, d_v=512, scale=0.07, q=FAKE, kv=FAKE, num_blocks=64,
                block_size=64, block_table=FAKE, max_blocks=32, seq_lens=FAKE, max_seq_len=2048)
    base.update(kw)
    return md.Problem(**base)


def dense_status(p, num_shards=1, interleave=1, shard_id=-1, out=FAKE, dtype=0, lse=FAKE):
    return lib.mla_decode_dense(ctypes.byref(p) if p is not None else None, num_shards, interleave,
                                shard_id, out, dtype, lse, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(kv=None), 1), (dict(block_table=None), 1), (dict(seq_lens=None), 1),
    (dict(d_qk=512), 3), (dict(d_v=576), 3), (dict(h_q=129), 3), (dict(Q=17), 3),
    (dict(B=0), 2), (dict(h_q=0), 2), (dict(block_size=48), 2), (dict(block_size=0), 2),
    (dict(max_seq_len=2049 + 31 * 64), 2), (dict(max_seq_len=0), 2), (dict(scale=float("nan")), 2),
    (dict(scale=0.0), 2), (dict(scale=-0.07), 2), (dict(group_rows=96), 2), (dict(group_rows=-64), 2),
    (dict(q=FAKE + 8), 2),
    (dict(kv_dtype=1), 1), (dict(kv_dtype=2, kv_scale=FAKE), 3), (dict(kv_dtype=-1), 3),
    (dict(kv_dtype=1, kv_scale=FAKE, group_rows=128), 3), (dict(kv_dtype=1, kv_scale=FAKE + 2), 2),
])
def test_dense_validation_statuses(kw, status):
    assert dense_status(problem(**kw)) == status


@pytest.mark.parametrize("h_q,Q,S", [(128, 1, 4096), (128, 1, 200000), (64, 2, 1000), (16, 1, 256)])
def test_plan_int8_cache_takes_64_row_groups(h_q, Q, S):
    p = problem(h_q=h_q, Q=Q, num_blocks=4096, max_blocks=4096, max_seq_len=S, kv_dtype=1, kv_scale=FAKE)
    plan = md.mla_plan_query(p, num_cus=256)
    assert plan["rows_per_group"] <= 64
    # the bf16 plan of the same problem may take 128 rows; the int8 one never does
    assert md.mla_plan_query(problem(h_q=h_q, Q=Q, num_blocks=4096, max_blocks=4096, max_seq_len=S,
                                     kv_dtype=1, kv_scale=FAKE, group_rows=64), num_cus=256) == plan


def test_dense_argument_statuses():
    assert dense_status(None) == 1
    assert dense_status(problem(), out=None) == 1
    assert dense_status(problem(), lse=None) == 1
    assert dense_status(problem(), dtype=7) == 2
    assert dense_status(problem(), num_shards=0) == 2
    assert dense_status(problem(), num_shards=4, interleave=0, dtype=1) == 2
    assert dense_status(problem(), num_shards=4, interleave=8, shard_id=4, dtype=1) == 2
    # sharded partials are fp32 only
    assert dense_status(problem(), num_shards=4, interleave=8, dtype=0) == 3
    # a plan that needs scratch without a workspace
    assert dense_status(problem()) == 1


def test_sparse_and_merge_argument_statuses():
    p = problem()
    f = lib.mla_decode_sparse
    assert f(ctypes.byref(p), None, 2048, 2048, 0, FAKE, 0, FAKE, None, 0, None) == 1
    assert f(ctypes.byref(p), FAKE, 0, 2048, 0, FAKE, 0, FAKE, None, 0, None) == 2
    assert f(ctypes.byref(p), FAKE, 2048, -1, 0, FAKE, 0, FAKE, None, 0, None) == 2
    assert f(ctypes.byref(p), FAKE, 70000, 70000, 0, FAKE, 0, FAKE, None, 0, None) == 2
    assert f(ctypes.byref(p), FAKE, 2048, 2048, 0, FAKE, 0, FAKE, FAKE, 16, None) == 4
    m = lib.mla_merge_lse
    assert m(None, FAKE, 2, 4, 512, FAKE, 1, FAKE, None) == 1
    assert m(FAKE, FAKE, 0, 4, 512, FAKE, 1, FAKE, None) == 2
    assert m(FAKE, FAKE, 2, 4, 510, FAKE, 1, FAKE, None) == 2
    assert m(FAKE, FAKE, 2, -1, 512, FAKE, 1, FAKE, None) == 2
    assert m(FAKE, FAKE, 2, 0, 512, FAKE, 1, FAKE, None) == 0  # nothing to do


def plan(p, **kw):
    return md.mla_plan_query(p, **kw)


def test_plan_fills_the_device_and_covers_every_tile():
    # sparse B=32 h=128 top_k=2048: 128-row groups would leave partitions of 4
    # tiles, so 64-row groups: 2 head chunks x 32 sequences = 64 units -> 4
    # partitions of 512 tokens
    pl = plan(problem(B=32, max_seq_len=32768, max_blocks=512), top_k=2048)
    assert (pl["q_per_group"], pl["rows_per_group"]) == (1, 64)
    assert (pl["units"], pl["splits"], pl["chunk"], pl["grid"]) == (64, 4, 512, 256)
    assert pl["workspace_bytes"] >= 4 * 32 * 128 * 512 * 4
    # dense B=32 S=4096: 128-row groups, 8 partitions of 8 tiles
    pl = plan(problem(B=32, max_seq_len=4096, max_blocks=64))
    assert pl["rows_per_group"] == 128
    assert (pl["splits"], pl["chunk"], pl["grid"]) == (8, 512, 256)
    # enough units: no partitions, no scratch
    pl = plan(problem(B=512, max_seq_len=4096, max_blocks=64))
    assert pl["splits"] == 1 and pl["workspace_bytes"] == 0
    # MTP: Q=2 x h=64 as one 64-row group per query token needs no partitions
    # (two tokens per 128-row group would); Q=4 x h=16 share one group
    pl = plan(problem(B=128, Q=2, h_q=64, max_seq_len=65536, max_blocks=1024), top_k=2048)
    assert pl["q_per_group"] == 1 and pl["rows_per_group"] == 64 and pl["units"] == 256
    pl = plan(problem(B=8, Q=4, h_q=16, max_seq_len=4096, max_blocks=64))
    assert pl["q_per_group"] == 4 and pl["rows_per_group"] == 64 and pl["units"] == 8
    pl = plan(problem(B=8, Q=4, h_q=32, max_seq_len=4096, max_blocks=64))
    assert pl["q_per_group"] == 2 and pl["rows_per_group"] == 64 and pl["units"] == 16
    # h_q = 96: a 64-head chunk and a 32-head chunk per query token
    pl = plan(problem(B=8, Q=2, h_q=96, max_seq_len=4096, max_blocks=64))
    assert pl["q_per_group"] == 1 and pl["rows_per_group"] == 64 and pl["units"] == 32
    # per-token index lists split the query tokens
    pl = plan(problem(B=128, Q=2, h_q=64, max_seq_len=65536, max_blocks=1024), top_k=2048,
              index_stride_q=2048)
    assert pl["q_per_group"] == 1 and pl["units"] == 256


@pytest.mark.parametrize("S,N,I", [(131072, 8, 64), (1000, 3, 7), (5, 8, 64), (64 * 8 * 3 + 17, 8, 64)])
def test_plan_shards_cover_their_positions(S, N, I):
    for r in list(range(N)) + [-1]:
        pl = plan(problem(B=8, max_seq_len=S, max_blocks=(S + 63) // 64), num_shards=N, interleave=I,
                  shard_id=r)
        counts = [sum(1 for p in range(S) if (p // I) % N == rr) for rr in range(N)]
        want = max(counts) if r < 0 else counts[r]
        assert pl["stream_len"] == want
        assert pl["splits"] * pl["chunk"] >= want and pl["chunk"] % 64 == 0
        assert (pl["splits"] - 1) * pl["chunk"] < max(want, 1)
        chunks = 128 // pl["rows_per_group"]  # 64-row groups: two head chunks of h_q = 128
        units = 8 * chunks * (N if r < 0 else 1)
        assert pl["grid"] == units * pl["splits"]


def test_plan_sparse_shards():
    # sparse x DCP: each shard streams its own part of the list, planned as an
    # even share of min(top_k, S) entries; the workspace holds the split lists
    pr = problem(B=8, max_seq_len=131072, max_blocks=2048)
    pl = plan(pr, top_k=2048, num_shards=8, interleave=64, shard_id=-1)
    assert pl["stream_len"] == 256
    assert pl["units"] == 8 * 8 * (128 // pl["rows_per_group"])  # sequences x shards x head chunks
    assert pl["grid"] == pl["units"] * pl["splits"]
    assert pl["splits"] * pl["chunk"] >= 256
    lists = 8 * 1 * 8 * 2048 * 4
    assert pl["workspace_bytes"] >= lists
    assert md.mla_workspace_size(pr, 8, 64, -1, 2048) == pl["workspace_bytes"]
    one = plan(pr, top_k=2048, num_shards=8, interleave=64, shard_id=3)
    assert one["stream_len"] == 256 and one["units"] == 8 * (128 // one["rows_per_group"])
    assert md.mla_workspace_size(pr, 8, 64, 3, 2048) >= 8 * 2048 * 4
    # short sequences bound the share: S = 1000 < top_k, 3 shards -> 334
    short = plan(problem(B=8, max_seq_len=1000, max_blocks=16), top_k=2048, num_shards=3, interleave=7)
    assert short["stream_len"] == 334
    # per-token lists (Q = 2) are sized for as well
    assert md.mla_workspace_size(problem(B=8, Q=2, max_seq_len=4096, max_blocks=64), 4, 64, -1, 512, 512) >= 8 * 2 * 4 * 512 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(num_shards=1), 2), (dict(num_shards=0), 2), (dict(shard_id=8), 2), (dict(shard_id=-2), 2),
    (dict(interleave=0), 2), (dict(indices=None), 1), (dict(out=None), 1), (dict(top_k=0), 2),
])
def test_sparse_dcp_argument_checks(kw, status):
    a = dict(indices=FAKE, top_k=64, num_shards=8, interleave=64, shard_id=-1, out=FAKE)
    a.update(kw)
    assert lib.mla_decode_sparse_dcp(ctypes.byref(problem()), a["indices"], a["top_k"], 64, 0,
                                     a["num_shards"], a["interleave"], a["shard_id"], a["out"], FAKE,
                                     None, 0, None) == status


def test_forced_group_rows_override_the_plan_and_reject_other_values():
    dense = dict(B=32, max_seq_len=4096, max_blocks=64)
    sparse = dict(B=32, max_seq_len=32768, max_blocks=512)
    pl = plan(problem(group_rows=64, **dense))
    assert (pl["rows_per_group"], pl["units"], pl["splits"], pl["chunk"]) == (64, 64, 4, 1024)
    pl = plan(problem(group_rows=128, **sparse), top_k=2048)
    assert (pl["rows_per_group"], pl["units"], pl["splits"], pl["chunk"]) == (128, 32, 8, 256)
    for bad in (-1, 1, 32, 96, 256):
        st = lib.mla_plan_query(ctypes.byref(problem(group_rows=bad, **sparse)), 1, 1, -1, 2048, 0, 256,
                                ctypes.byref(md.Plan()))
        assert st == 2, bad
    # the default picks per problem
    assert plan(problem(**dense))["rows_per_group"] == 128
    assert plan(problem(**sparse), top_k=2048)["rows_per_group"] == 64


@pytest.mark.parametrize("args,status", [
    (dict(T=-1), 2), (dict(num_slots=0), 2), (dict(num_slots=1 << 31), 2),
    (dict(num_shards=0), 2), (dict(num_shards=2, interleave=0), 2), (dict(num_shards=2, shard_id=2), 2),
    (dict(num_shards=2, shard_id=-1), 2), (dict(rows=None), 1), (dict(slots=None), 1), (dict(kv=None), 1),
    (dict(num_shards=2, positions=None), 1), (dict(rows=FAKE + 8), 2), (dict(kv=FAKE + 4), 2),
    (dict(T=0, rows=None, slots=None, kv=None), 0),
])
def test_kv_write_argument_checks(args, status):
    a = dict(rows=FAKE, slots=FAKE, T=10, kv=FAKE, num_slots=100, positions=FAKE, num_shards=1,
             interleave=1, shard_id=0)
    a.update(args)
    assert lib.mla_kv_write(a["rows"], a["slots"], a["T"], a["kv"], a["num_slots"], a["positions"],
                            a["num_shards"], a["interleave"], a["shard_id"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(scores=None), 1), (dict(seq_lens=None), 1), (dict(out=None), 1), (dict(B=0), 2), (dict(Q=0), 2),
    (dict(Q=17), 2), (dict(max_len=0), 2), (dict(top_k=0), 2), (dict(top_k=65537), 2), (dict(stride_b=-1), 2),
    (dict(stride_q=-1), 2),
])
def test_topk_argument_checks(kw, status):
    a = dict(scores=FAKE, stride_b=4096, stride_q=2048, seq_lens=FAKE, B=2, Q=2, max_len=2048, top_k=64, out=FAKE)
    a.update(kw)
    assert lib.mla_topk_select(a["scores"], a["stride_b"], a["stride_q"], a["seq_lens"], a["B"], a["Q"],
                               a["max_len"], a["top_k"], a["out"], None) == status


def _sweep_cases():
    """(problem kwargs, num_shards, interleave, shard_id, top_k, index_stride_q) over
    sizes around tile and block boundaries, every interleave class (smaller than,
    equal to and larger than a tile, larger than the sequence), each shard and
    all shards, dense and sparse, shared and per-token lists, both group shapes."""
    cases = []
    for B in (1, 4, 32):
        for S in (300, 2049, 4096, 70001):
            mb = (S + 63) // 64
            for Q, h in ((1, 128), (2, 64), (4, 16)):
                for gr in (0, 64, 128):
                    pk = dict(B=B, Q=Q, h_q=h, max_seq_len=S, max_blocks=mb, num_blocks=mb * B + 8,
                              group_rows=gr)
                    cases.append((pk, 1, 1, -1, 0, 0))
                    for k in (64, 2048):
                        cases.append((pk, 1, 1, -1, k, 0))
                        cases.append((pk, 1, 1, -1, k, k))
                    for N in (2, 4, 8):
                        for I in (1, 7, 64, 128, 512, 1024):
                            for r in (-1, 0, N - 1):
                                cases.append((pk, N, I, r, 0, 0))
                                cases.append((pk, N, I, r, 2048, 2048 if Q > 1 else 0))
    return cases


def test_workspace_size_is_the_plan_size_everywhere():
    """mla_workspace_size gives exactly what the decode call's plan needs, for
    every interleave (dense DCP shard streams depend on it), shard choice, list
    length and list stride."""
    bad = []
    for pk, N, I, r, k, sq in _sweep_cases():
        p = problem(**pk)
        pl = plan(p, num_shards=N, interleave=I, shard_id=r, top_k=k, index_stride_q=sq, num_cus=256)
        ws = md.mla_workspace_size(p, N, I, r, k, sq)
        if ws != pl["workspace_bytes"]:
            bad.append((pk, N, I, r, k, sq, ws, pl["workspace_bytes"]))
    assert not bad, f"{len(bad)} mismatches, first {bad[:3]}"


@pytest.mark.parametrize("S,N,I,B", [(2049, 4, 1024, 1), (2049, 8, 512, 4), (300, 2, 512, 1)])
def test_workspace_size_covers_large_interleaves(S, N, I, B):
    """Shapes whose shard streams are long only because the interleave is large:
    one run of I tokens holds most of the sequence."""
    p = problem(B=B, h_q=16 if S == 300 else 128, max_seq_len=S, max_blocks=(S + 63) // 64)
    need = plan(p, num_shards=N, interleave=I, shard_id=-1, num_cus=256)["workspace_bytes"]
    assert need > 0
    assert md.mla_workspace_size(p, N, I, -1, 0, 0) == need


def test_workspace_size_rejects_bad_arguments():
    invalid = ctypes.c_size_t(-1).value
    p = problem()
    assert lib.mla_workspace_size(ctypes.byref(p), 4, 0, -1, 0, 0) == invalid      # interleave 0
    assert lib.mla_workspace_size(ctypes.byref(p), 4, 64, 4, 0, 0) == invalid      # shard out of range
    assert lib.mla_workspace_size(ctypes.byref(p), 1, 1, -1, -5, 0) == invalid     # negative top_k
    assert lib.mla_workspace_size(ctypes.byref(p), 1, 1, -1, 64, -1) == invalid    # negative stride
    assert lib.mla_workspace_size(ctypes.byref(problem(d_qk=512)), 1, 1, -1, 0, 0) == invalid


def _usable_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_usable_gpu(), reason="checks the status where no GPU is visible")
def test_valid_calls_without_a_device_return_mla_err_device():
    """Every argument is valid, so the only thing left to fail is the device:
    the call says so (MLA_ERR_DEVICE) instead of reporting a launch failure."""
    p = problem(B=512, max_seq_len=4096, max_blocks=64)   # no partitions: needs no workspace
    assert plan(p)["workspace_bytes"] == 0
    assert lib.mla_decode_dense(ctypes.byref(p), 1, 1, -1, FAKE, 0, FAKE, None, 0, None) == 6
    assert lib.mla_decode_sparse(ctypes.byref(p), FAKE, 64, 64, 0, FAKE, 0, FAKE, None, 0, None) == 6
    assert lib.mla_merge_lse(FAKE, FAKE, 2, 4, 512, FAKE, 1, FAKE, None) == 6
    assert lib.mla_topk_select(FAKE, 4096, 2048, FAKE, 2, 2, 2048, 64, FAKE, None) == 6
    assert lib.mla_kv_write(FAKE, FAKE, 10, FAKE, 100, FAKE, 1, 1, 0, None) == 6


def test_noalloc_entry_point_checks_arguments_and_its_scratch_limit():
    """The allocation-free sparse call validates like mla_decode_sparse and
    rejects, before touching the device, a plan needing more than its fixed
    buffer (mla_workspace_size gives the amount)."""
    f = lib.mla_decode_sparse_noalloc
    p = problem()
    assert f(ctypes.byref(p), None, 2048, 2048, 0, FAKE, 0, FAKE, None) == 1
    assert f(ctypes.byref(p), FAKE, 0, 2048, 0, FAKE, 0, FAKE, None) == 2
    assert f(ctypes.byref(p), FAKE, 2048, -1, 0, FAKE, 0, FAKE, None) == 2
    assert f(ctypes.byref(p), FAKE, 2048, 2048, 0, FAKE, 7, FAKE, None) == 2
    assert f(ctypes.byref(problem(d_qk=512)), FAKE, 2048, 2048, 0, FAKE, 0, FAKE, None) == 3
    big = problem(B=8, Q=4, h_q=128, max_seq_len=65536, max_blocks=1024, num_blocks=16384)
    need = md.mla_workspace_size(big, 1, 1, -1, 4096, 0)
    assert need > (64 << 20)
    assert f(ctypes.byref(big), FAKE, 4096, 4096, 0, FAKE, 0, FAKE, None) == 7
    assert "64 MiB" in md.mla_status_string(7)
