"""GPU parity of the top-k selection (mla_topk_select) against oracle/topk.py:
the selected positions must match exactly, at small and full sizes, on rows
with heavy ties, NaN, infinities and signed zeros, short and empty rows; and the
selection feeds the sparse decode directly."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
from oracle import topk  # noqa: E402
from latent_decode_attention_amd import mla_decode as md  # noqa: E402
from latent_decode_attention_amd import workloads as W  # noqa: E402
from latent_decode_attention_amd.device import upload, run  # noqa: E402

pytestmark = pytest.mark.gpu


def gpu_select(x, top_k=None):
    s = torch.from_numpy(x.scores).cuda()
    sl = torch.from_numpy(x.seq_lens).cuda()
    out = md.mla_topk_select(s, sl, top_k or x.top_k)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("B,Q,lens,k", [
    (1, 1, [1], 1), (1, 1, [5], 8), (2, 1, [3000, 1024], 1024), (3, 2, [5000, 100, 2049], 2048),
    (4, 4, [70, 4097, 1, 2052], 2048), (2, 1, [131072, 99999], 2048), (2, 3, [40000, 3], 1), (1, 1, [65536], 65536),
    # rows of one segment with k > 4096: no per-thread lower bound, every key counted
    (1, 1, [32768], 20000), (2, 1, [30000, 9000], 5000), (1, 2, [32768], 32766),
])
def test_topk_matches_the_oracle(B, Q, lens, k):
    x = W.make_topk_scores(B, Q, lens, k, seed=B * 100 + Q + k)
    assert np.array_equal(gpu_select(x), topk.select(x.scores, x.seq_lens, k))


@pytest.mark.parametrize("zero_frac", [0.0, 0.9, 1.0])
def test_topk_with_heavy_ties(zero_frac):
    x = W.make_topk_scores(3, 1, [20000, 4096, 2049], 2048, seed=7, zero_frac=zero_frac)
    assert np.array_equal(gpu_select(x), topk.select(x.scores, x.seq_lens, 2048))


def test_topk_special_values():
    g = np.random.default_rng(11)
    x = W.make_topk_scores(4, 1, [9000] * 4, 300, seed=12)
    vals = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-45, -1e-45],
                    dtype=np.float32)
    x.scores[0, 0, :9000] = g.choice(vals, 9000)                  # only special values
    x.scores[1, 0, :9000] = np.nan                                # all NaN: first 300 positions
    x.scores[2, 0, :9000] = np.where(g.random(9000) < 0.5, -0.0, 0.0)  # signed zeros are one value
    x.scores[3, 0, :9000] = -np.inf
    x.scores[3, 0, g.choice(9000, 200, replace=False)] = np.nan   # 8800 x -inf, 200 x NaN
    got = gpu_select(x)
    assert np.array_equal(got, topk.select(x.scores, x.seq_lens, 300))
    assert got[1, 0].tolist() == list(range(300)) and got[2, 0].tolist() == list(range(300))


def test_topk_at_the_bench_size():
    # The headline sparse shape: 32 sequences of 32768 positions, top 2048.
    x = W.make_topk_scores(32, 1, [32768] * 32, 2048, seed=1009)
    assert np.array_equal(gpu_select(x), topk.select(x.scores, x.seq_lens, 2048))


def test_selected_positions_drive_the_sparse_decode():
    # indexer scores -> top-k -> sparse decode, against the oracle's selection fed
    # to the oracle's decode
    w = W.make_workload("topk_decode", 3, 2, 64, [3000, 700, 2049], 16, seed=81)
    x = W.make_topk_scores(3, 2, w.seq_lens, 512, seed=82)
    sel = gpu_select(x)
    want = topk.select(x.scores, x.seq_lens, 512)
    assert np.array_equal(sel, want)
    w.indices, w.top_k, w.index_stride_b, w.index_stride_q = want, 512, 2 * 512, 512
    d = upload(w)
    out, lse = run(d, out_dtype=torch.float32, indices=torch.from_numpy(sel).cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.sparse(w)
    assert np.abs(out.cpu().numpy().astype(np.float64).reshape(ro.shape) - ro).max() <= 1e-2
    assert np.abs(lse.cpu().numpy().astype(np.float64).reshape(rl.shape) - rl).max() <= 1e-3


def test_topk_of_unaligned_strided_rows():
    # rows start 4 bytes past a 16-byte boundary and are padded to a larger
    # stride: the scalar-load path, and strides taken from the tensor
    x = W.make_topk_scores(3, 2, [9000, 3000, 40000], 1000, seed=21)
    B, Q, n = x.scores.shape
    wide = np.full((B, Q, n + 7), np.inf, dtype=np.float32)
    wide[:, :, 1:n + 1] = x.scores
    s = torch.from_numpy(wide).cuda()[:, :, 1:n + 1]
    assert s.data_ptr() % 16 == 4
    got = md.mla_topk_select(s, torch.from_numpy(x.seq_lens).cuda(), 1000)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), topk.select(x.scores, x.seq_lens, 1000))


@pytest.mark.parametrize("B,lens,k", [(4, [32768, 30000, 5000, 2049], 2048), (2, [32768, 9000], 300),
                                      (32, [32768] * 32, 2048), (2, [32767, 20001], 6000)])
def test_topk_of_full_precision_scores(B, lens, k):
    # fp32 scores using all 32 bits (the other cases hold bf16 values): the
    # low halves of the keys decide the last chosen score, and the zeros and
    # the +inf past each row are kept
    x = W.make_topk_scores(B, 1, lens, k, seed=31 + B)
    full = np.random.default_rng(33 + B).standard_normal(x.scores.shape).astype(np.float32)
    x.scores[...] = np.where(np.isinf(x.scores) | (x.scores == 0), x.scores, full)
    assert (x.scores.view(np.uint32) & 0xffff).any()
    assert np.array_equal(gpu_select(x), topk.select(x.scores, x.seq_lens, k))
