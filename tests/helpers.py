"""Test helpers: hand-built workloads from logical (unpaged) per-sequence rows.

Building the logical content first and paging it here, with a permutation the
test chooses, lets a test compare the oracle (which reads the paged layout
through the block table) with computations on the logical rows.
"""
from __future__ import annotations

import numpy as np

from latent_decode_attention_amd.workloads import (BF16_NAN, D_QK, D_V, Workload,
                                                   f32_to_bf16_bits, bf16_bits_to_f32)


def bf16(x):
    """bf16 bits of x (a scalar in gives a numpy scalar out)."""
    a = np.asarray(x, dtype=np.float32)
    r = f32_to_bf16_bits(a).reshape(a.shape)
    return r[()] if a.ndim == 0 else r


def f64(bits) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def paged(logical, block_size: int, rng: np.random.Generator, spare: int = 2):
    """Page per-sequence logical rows [S_b, 576] (uint16) into a permuted block pool."""
    nblk = [(len(x) + block_size - 1) // block_size for x in logical]
    used = sum(nblk)
    num_blocks = used + spare
    kv = np.full((num_blocks, block_size, D_QK), BF16_NAN, dtype=np.uint16)
    perm = rng.permutation(num_blocks)
    maxb = max(1, max(nblk))
    bt = np.full((len(logical), maxb), perm[-1] if spare else perm[0], dtype=np.int32)
    o = 0
    for b, x in enumerate(logical):
        for j in range(nblk[b]):
            phys = perm[o]
            o += 1
            bt[b, j] = phys
            seg = x[j * block_size:(j + 1) * block_size]
            kv[phys, :len(seg)] = seg
    return kv, bt


def workload(q_bits, logical, block_size=16, scale=1.0 / np.sqrt(192.0), seed=0, spare=2,
             **kw) -> Workload:
    """Workload from q bits [B,Q,h,576] and logical rows per sequence."""
    rng = np.random.default_rng(seed)
    kv, bt = paged(logical, block_size, rng, spare)
    B, Q, h, _ = q_bits.shape
    return Workload(name="handmade", B=B, Q=Q, h_q=h, scale=float(scale), block_size=block_size,
                    q=np.ascontiguousarray(q_bits), kv=kv, block_table=bt,
                    seq_lens=np.array([len(x) for x in logical], dtype=np.int32), **kw)


def random_rows(rng, n, cols=D_QK, std=1.0):
    return bf16(rng.standard_normal((n, cols)) * std)


def validate_device_inputs(w: Workload) -> dict:
    """Test-only check of the device data a decode call trusts without looking.

    The library validates shapes on the host but not the contents of seq_lens,
    block_table and indices: an attended position whose block id is outside
    [0, num_blocks) is skipped on the device, and list entries outside
    [0, pos(b, q)] are dropped.  This reports what a caller should have ruled
    out: `bad_seq_lens` (outside [Q, max_blocks * block_size]), `bad_blocks`
    ((b, logical block) pairs below S_b whose id is out of range), and for
    sparse lists `out_of_range` (entries that are neither -1 padding nor in
    [0, S_b - 1]: no query token can attend them), `causal_masked` (entries in
    range but past pos(b, q), dropped for that token only: normal for a list
    shared by the Q tokens) and `duplicates` (positions listed twice for one
    query token).
    """
    num_blocks, bs = w.kv.shape[0], w.block_size
    rep = dict(bad_seq_lens=[], bad_blocks=[], out_of_range=0, causal_masked=0, padding=0, duplicates=0)
    for b in range(w.B):
        S = int(w.seq_lens[b])
        if S < w.Q or S > w.block_table.shape[1] * bs:
            rep["bad_seq_lens"].append(b)
            continue
        for j in range((S + bs - 1) // bs):
            blk = int(w.block_table[b, j])
            if blk < 0 or blk >= num_blocks:
                rep["bad_blocks"].append((b, j))
        if w.indices is None:
            continue
        flat = np.asarray(w.indices).reshape(-1)
        for q in range(w.Q):
            start = b * w.index_stride_b + q * w.index_stride_q
            lst = flat[start:start + w.top_k].astype(np.int64)
            pos = S - w.Q + q
            rep["padding"] += int(np.count_nonzero(lst == -1))
            rep["out_of_range"] += int(np.count_nonzero((lst != -1) & ((lst < 0) | (lst >= S))))
            rep["causal_masked"] += int(np.count_nonzero((lst > pos) & (lst < S)))
            valid = lst[(lst >= 0) & (lst <= pos)]
            rep["duplicates"] += int(valid.size - np.unique(valid).size)
    return rep


def device_inputs_ok(w: Workload) -> bool:
    rep = validate_device_inputs(w)
    return not rep["bad_seq_lens"] and not rep["bad_blocks"] and rep["out_of_range"] == 0
