"""TEST INFRASTRUCTURE ONLY: plain CPU reference for the indexer's top-k selection.

Only ``tests/`` and the CPU-baseline leg of ``bench.py`` may import this module.
The product library never links, loads or calls it, and it shares no code with
the HIP path.

The sparse attention reads, for every query token, the positions an indexer
selected: the top-2048 of the indexer's scores over the sequence ("vllm-ascend PR
#18870 解读：FlashComm1 的'假开启'与 SP 归位", §4.5, the design-benefit table;
"RFC: Context Parallel Modeling for DeepSeek-Style Attention", §3.3, where the
top-k query side of the fused indexer is modelled separately from its scoring).
The pages fix neither the tie rule nor the order of the result; the readings
used here:

* row (b, q) scores positions [0, L) with L = seq_lens[b] - Q + q + 1, the causal
  limit of query token q (clipped to [0, max_len]);
* a score ranks above another when it is larger; NaN ranks below every number;
  -0 and +0 are equal; equal scores rank by position, lower first;
* the result is the min(top_k, L) best positions, in ascending position order,
  padded with -1 to top_k.

Under this total order the selected set is unique, so the GPU result can be
compared position for position.
"""
from __future__ import annotations

import numpy as np


def row_length(seq_len: int, Q: int, q: int, max_len: int) -> int:
    """Positions query token q of Q may select: those up to its own, S - Q + q."""
    return int(min(max(seq_len - Q + q + 1, 0), max_len))


def select_row(scores: np.ndarray, top_k: int) -> np.ndarray:
    """Top-k positions of one row of scores (all of it valid), ascending, -1 padded."""
    L = scores.shape[0]
    s = scores.astype(np.float64)
    is_nan = np.isnan(s)
    value = np.where(is_nan, 0.0, s) + 0.0          # -0 -> +0; NaN handled by is_nan
    pos = np.arange(L)
    # Rank: numbers before NaN, then larger value first, then lower position first
    # (np.lexsort sorts by its last key first).
    ranked = np.lexsort((pos, -value, is_nan))
    chosen = np.sort(ranked[:min(top_k, L)])
    out = np.full(top_k, -1, dtype=np.int32)
    out[:chosen.shape[0]] = chosen
    return out


def select(scores: np.ndarray, seq_lens: np.ndarray, top_k: int) -> np.ndarray:
    """scores: float32 [B, Q, max_len]; seq_lens: int [B].  Returns int32 [B, Q, top_k]."""
    B, Q, max_len = scores.shape
    out = np.empty((B, Q, top_k), dtype=np.int32)
    for b in range(B):
        for q in range(Q):
            L = row_length(int(seq_lens[b]), Q, q, max_len)
            out[b, q] = select_row(scores[b, q, :L], top_k)
    return out
