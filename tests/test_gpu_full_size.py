"""GPU parity at the full sizes of the measured workloads, on every output row.

Each test builds its workload once, computes the fp64 oracle once, and runs the
HIP path (in the launch configuration the benchmark times, plus the other
work-group shape) against it: all rows of the unsharded outputs, every shard of
the DCP workloads and their merge.  The largest errors are recorded per
workload (tests/parity.py) for the results table.

Workloads (seeded, shapes of the measured decode cases):
  2  dense, B32 Q1 h128 S4096, paged bs64
  3  sparse top-2048, B32 Q1 h128 S32768 (3 rows keep 1500 entries)
  4  dense DCP, B8 Q1 h128 S131072, 8 shards interleaved by 64, merged
  5  MTP sparse, B128 Q2 h64, S log-uniform in [1k, 64k], RoPE-column outliers
  6  dense, B32 Q1 h128 S32768
  7  sparse DCP, B8 Q1 h128 S131072 top-2048, 8 shards, merged
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import parity  # noqa: E402
from latent_decode_attention_amd import mla_decode as md  # noqa: E402
from latent_decode_attention_amd import workloads as W  # noqa: E402
from latent_decode_attention_amd.device import run, upload  # noqa: E402

pytestmark = pytest.mark.gpu

SHAPES = (0, 64, 128)  # the planner's choice (what the benchmark times), then both forced shapes


def _shapes(w):
    # int8 caches run with 64-row groups only; every shape otherwise
    return (0,) if w.kv8 is not None else SHAPES


@pytest.fixture(autouse=True)
def reset_shape():
    yield
    md.GROUP_ROWS = 0


def _label(cfg, gr, out_dtype, extra=""):
    return f"cfg{cfg}{extra}/rows{gr or 'plan'}/{'bf16' if out_dtype == torch.bfloat16 else 'fp32'}"


@pytest.mark.parametrize("cfg", [2, 3, 5, 6])
def test_full_size_unsharded_every_row(cfg):
    w = W.PRESETS[cfg]()
    d = upload(w)
    ro, rl = oracle.sparse(w) if w.indices is not None else oracle.dense(w)
    for gr in _shapes(w):
        md.GROUP_ROWS = gr
        for out_dtype in (torch.bfloat16, torch.float32):
            print(f"[full] cfg {cfg} rows {gr} {out_dtype}", flush=True)
            out, lse = run(d, out_dtype=out_dtype)
            torch.cuda.synchronize()
            lab = _label(cfg, gr, out_dtype)
            parity.check_o(out, ro, f"{w.name} rows {gr}", label=lab)
            parity.check_lse(lse, rl, f"{w.name} rows {gr}", label=lab)
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", [4, 7])
def test_full_size_dcp_every_shard_and_merge(cfg):
    w = W.PRESETS[cfg]()
    d = upload(w)
    N, I = w.num_shards, w.interleave
    if w.indices is not None:
        shard_ref = [oracle.sparse(w, num_shards=N, interleave=I, shard_id=r) for r in range(N)]
        ro, rl = oracle.sparse(w)
    else:
        shard_ref = [oracle.dense(w, num_shards=N, interleave=I, shard_id=r) for r in range(N)]
        ro, rl = oracle.dense(w)
    for gr in SHAPES:
        md.GROUP_ROWS = gr
        print(f"[full] cfg {cfg} rows {gr}", flush=True)
        parts, lses = run(d)
        torch.cuda.synchronize()
        for r in range(N):
            lab = _label(cfg, gr, torch.float32, "-shards")
            parity.check_o(parts[r], shard_ref[r][0], f"{w.name} shard {r} rows {gr}", label=lab)
            parity.check_lse(lses[r], shard_ref[r][1], f"{w.name} shard {r} rows {gr}", label=lab)
        for out_dtype in (torch.bfloat16, torch.float32):
            merged, mlse = md.mla_merge_lse(parts, lses, out_dtype=out_dtype)
            torch.cuda.synchronize()
            lab = _label(cfg, gr, out_dtype, "-merged")
            parity.check_o(merged, ro, f"{w.name} merged rows {gr}", label=lab)
            parity.check_lse(mlse, rl, f"{w.name} merged rows {gr}", label=lab)
    del d, parts, lses
    torch.cuda.empty_cache()


def test_full_size_int8_cache_every_row():
    """The headline sparse workload over the int8 cache (factor x code per row)."""
    w = W.int8_cache(W.PRESETS[3]())
    d = upload(w)
    ro, rl = oracle.sparse(w)
    for out_dtype in (torch.bfloat16, torch.float32):
        out, lse = run(d, out_dtype=out_dtype)
        torch.cuda.synchronize()
        lab = _label(3, 0, out_dtype, "-int8")
        parity.check_o(out, ro, f"{w.name} int8", label=lab)
        parity.check_lse(lse, rl, f"{w.name} int8", label=lab)
