"""GPU: the allocation-free sparse entry point (fixed device scratch) against
mla_decode_sparse with a caller workspace, through the C ABI: the same plan and
kernels, so the results agree bit for bit (and meet the contract bar against the
oracle); two calls in a row, the second smaller, on one device's scratch."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import parity  # noqa: E402
from latent_decode_attention_amd import mla_decode as md  # noqa: E402
from latent_decode_attention_amd import workloads as W  # noqa: E402
from latent_decode_attention_amd.device import upload  # noqa: E402

pytestmark = pytest.mark.gpu


def _both(w, out_dtype):
    d = upload(w)
    kw = dict(scale=w.scale, max_seq_len=w.max_seq_len, top_k=w.top_k, index_stride_b=w.index_stride_b,
              index_stride_q=w.index_stride_q)
    ref = md.mla_decode_sparse(d.q, d.kv, d.block_table, d.seq_lens, d.indices, out_dtype=out_dtype, **kw)
    out = torch.full((w.B, w.Q, w.h_q, 512), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((w.B, w.Q, w.h_q), float("nan"), dtype=torch.float32, device="cuda")
    md.mla_decode_sparse_noalloc(d.q, d.kv, d.block_table, d.seq_lens, d.indices, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    return ref, (out, lse)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_noalloc_matches_the_workspace_call_twice_in_a_row(out_dtype):
    # first the headline sparse workload (4 split-KV partitions: its partials fill
    # 34 MB of the scratch), then a smaller call whose partials are laid out
    # differently over the same scratch (stale contents from the first call)
    big = W.PRESETS[3]()
    small = W.make_workload("noalloc_small", 3, 2, 64, [3000, 700, 4097], 64, seed=77, top_k=512,
                            short_rows=1, short_valid=100)
    for w in (big, small):
        d = upload(w)
        pl = md.mla_plan_query(md.make_problem(d.q, d.kv, d.block_table, d.seq_lens, w.scale, w.max_seq_len),
                               top_k=w.top_k, index_stride_q=w.index_stride_q)
        assert pl["splits"] > 1 and pl["workspace_bytes"] <= (64 << 20)
        (ro, rl), (o, l) = _both(w, out_dtype)
        assert torch.equal(ro, o) and torch.equal(rl, l), w.name
    ref_o, ref_l = oracle.sparse(small)
    parity.check_o(o, ref_o, "noalloc small")
    parity.check_lse(l, ref_l, "noalloc small")


def test_noalloc_without_partitions_and_over_the_limit():
    # a plan with no partitions touches no scratch at all
    w = W.make_workload("noalloc_nosplit", 300, 1, 64, [600] * 300, 64, seed=78, top_k=256)
    (ro, rl), (o, l) = _both(w, torch.bfloat16)
    assert torch.equal(ro, o) and torch.equal(rl, l)
    # a call that would need more than the fixed buffer is refused, nothing runs
    q = torch.zeros((8, 4, 128, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((16384, 64, 576), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((8, 1024), dtype=torch.int32, device="cuda")
    sl = torch.full((8,), 65536, dtype=torch.int32, device="cuda")
    idx = torch.zeros((8, 4096), dtype=torch.int32, device="cuda")
    out = torch.zeros((8, 4, 128, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((8, 4, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(md.MlaError) as e:
        md.mla_decode_sparse_noalloc(q, kv, bt, sl, idx, scale=0.07, max_seq_len=65536, out=out, lse=lse)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
