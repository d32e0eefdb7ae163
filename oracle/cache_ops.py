"""TEST INFRASTRUCTURE ONLY: plain CPU references for the cache-side operations.

Only ``tests/`` and the CPU-baseline leg of ``bench.py`` may import this module.
The product library never links, loads or calls it, and it shares no code with
the HIP path.  Plain numpy on whole arrays of raw bits, one token at a time
where the definition is per token.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def shard_of(positions: np.ndarray, num_shards: int, interleave: int) -> np.ndarray:
    """DCP owner of each position: tokens are interleaved over the ranks in runs of
    `interleave` ("RFC: MsModeling 支持 Decode Context Parallel 仿真", §2.1.4.1:
    cp_kv_cache_interleave_size)."""
    return (positions // interleave) % num_shards


def kv_write(kv_bits: np.ndarray, rows_bits: np.ndarray, slot_mapping: np.ndarray,
             positions: Optional[np.ndarray] = None, num_shards: int = 1, interleave: int = 1,
             shard_id: int = 0) -> np.ndarray:
    """The latent cache after storing each token's row at its slot.

    kv_bits: uint16 [num_slots, 576] (the cache's bf16 bits, flattened over blocks);
    rows_bits: uint16 [T, 576]; slot_mapping: int32 [T].  Follows the DCP page's
    table A (§2.1.4.1): the MLA cache [N_blk, block_size, D] addressed through the
    int32 slot_mapping; a token is stored only when its slot lies in the cache and,
    with DCP, when this rank owns its position.  Returns a new array.
    """
    out = kv_bits.copy()
    num_slots = out.shape[0]
    for t in range(rows_bits.shape[0]):
        slot = int(slot_mapping[t])
        if slot < 0 or slot >= num_slots:
            continue
        if num_shards > 1:
            p = int(positions[t])
            if p < 0 or (p // interleave) % num_shards != shard_id:
                continue
        out[slot] = rows_bits[t]
    return out
