"""GPU parity of the latent-cache write (mla_kv_write) against the plain
reference in oracle/cache_ops.py: the cache's bytes must match exactly."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from oracle import cache_ops  # noqa: E402
from latent_decode_attention_amd import mla_decode as md  # noqa: E402
from latent_decode_attention_amd import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a).view(dtype)).cuda()


def _run(kv_bits, x, **kw):
    kv = _dev(kv_bits, np.int16).view(torch.bfloat16)
    pos = _dev(x.positions, np.int32) if kw.get("num_shards", 1) > 1 else None
    md.mla_kv_write(_dev(x.rows, np.int16).view(torch.bfloat16), _dev(x.slots, np.int32), kv,
                    positions=pos, **kw)
    torch.cuda.synchronize()
    return kv.view(torch.int16).cpu().numpy().view(np.uint16)


def _cache(num_slots, seed):
    return np.random.default_rng(seed).integers(0, 1 << 16, size=(num_slots, W.D_QK), dtype=np.uint16)


@pytest.mark.parametrize("T,num_slots", [(1, 3), (37, 64 * 16), (1000, 4096), (5000, 64 * 1024)])
def test_kv_write_matches_the_reference(T, num_slots):
    x = W.make_kv_write_inputs(T, num_slots, seed=T)
    kv = _cache(num_slots, T + 1)
    assert np.array_equal(_run(kv, x), cache_ops.kv_write(kv, x.rows, x.slots))


def test_kv_write_of_zero_tokens_changes_nothing():
    x = W.make_kv_write_inputs(0, 100, seed=2)
    kv = _cache(100, 3)
    assert np.array_equal(_run(kv, x), kv)


@pytest.mark.parametrize("shard_id", range(8))
def test_kv_write_one_interleaved_shard(shard_id):
    x = W.make_kv_write_inputs(3000, 8192, seed=40)
    kv = _cache(8192, 41)
    want = cache_ops.kv_write(kv, x.rows, x.slots, x.positions, 8, 64, shard_id)
    assert np.array_equal(_run(kv, x, num_shards=8, interleave=64, shard_id=shard_id), want)


def test_kv_write_at_the_bench_size():
    # 32768 prefill tokens into a 64k-slot cache: the measured configuration.
    x = W.make_kv_write_inputs(32768, 65536, seed=1007)
    kv = _cache(65536, 1008)
    assert np.array_equal(_run(kv, x), cache_ops.kv_write(kv, x.rows, x.slots))


def test_decode_reads_the_rows_the_write_stored():
    # The last 40 positions of each sequence are overwritten with NaN, then stored
    # back by mla_kv_write through slots block_table[b, p / bs] * bs + p % bs (two
    # interleaved DCP shards, each storing its own tokens): the decode of the
    # restored cache must match the oracle on the original cache.
    import oracle
    from latent_decode_attention_amd.device import upload, run
    w = W.make_workload("kvw_decode", 2, 1, 16, [300, 170], 16, seed=21)
    ref_o, ref_l = oracle.dense(w)
    bs = w.block_size
    flat = w.kv.reshape(-1, W.D_QK)
    rows, slots, pos = [], [], []
    for b, S in enumerate(w.seq_lens):
        for p in range(S - 40, S):
            slot = int(w.block_table[b, p // bs]) * bs + p % bs
            rows.append(flat[slot].copy())
            slots.append(slot)
            pos.append(p)
    rows, slots, pos = np.stack(rows), np.array(slots, np.int32), np.array(pos, np.int32)
    w.kv = w.kv.copy()
    w.kv.reshape(-1, W.D_QK)[slots] = W.BF16_NAN
    d = upload(w)
    for r in range(2):
        md.mla_kv_write(_dev(rows, np.int16).view(torch.bfloat16), _dev(slots, np.int32),
                        d.kv.view(-1, W.D_QK), positions=_dev(pos, np.int32), num_shards=2, interleave=16,
                        shard_id=r)
    out, lse = run(d, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.abs(out.cpu().numpy().astype(np.float64).reshape(ref_o.shape) - ref_o).max() <= 1e-2
    assert np.abs(lse.cpu().numpy().astype(np.float64).reshape(ref_l.shape) - ref_l).max() <= 1e-3
