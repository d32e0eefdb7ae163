"""Device-memory plumbing: move a seeded Workload's arrays into torch GPU tensors."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .workloads import Workload


@dataclass
class DeviceWorkload:
    q: torch.Tensor            # bf16 [B, Q, h_q, 576]
    kv: torch.Tensor           # bf16 [num_blocks, block_size, 576], or int8 with kv_scale
    block_table: torch.Tensor  # int32 [B, max_blocks]
    seq_lens: torch.Tensor     # int32 [B]
    indices: Optional[torch.Tensor]  # int32, flat as the workload stores it
    w: Workload
    kv_scale: Optional[torch.Tensor] = None  # fp32 [num_blocks, block_size] (int8 cache)


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """Raw bf16 bits (uint16) -> a bf16 tensor on `device` with the same bytes."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def upload(w: Workload, device="cuda") -> DeviceWorkload:
    idx = None
    if w.indices is not None:
        idx = torch.from_numpy(np.ascontiguousarray(w.indices, dtype=np.int32)).to(device)
    if w.kv8 is not None:
        kv = torch.from_numpy(np.ascontiguousarray(w.kv8, dtype=np.int8)).to(device)
        kv_scale = torch.from_numpy(np.ascontiguousarray(w.kv_scale, dtype=np.float32)).to(device)
    else:
        kv, kv_scale = bf16_tensor(w.kv, device), None
    return DeviceWorkload(
        q=bf16_tensor(w.q, device), kv=kv,
        block_table=torch.from_numpy(np.ascontiguousarray(w.block_table, dtype=np.int32)).to(device),
        seq_lens=torch.from_numpy(np.ascontiguousarray(w.seq_lens, dtype=np.int32)).to(device),
        indices=idx, w=w, kv_scale=kv_scale)


def run(d: DeviceWorkload, out_dtype=torch.bfloat16, shard_id: Optional[int] = None, workspace=None,
        indices: Optional[torch.Tensor] = None, stream=None):
    """Call the library entry point that the workload describes."""
    from . import mla_decode as md
    w = d.w
    if w.indices is not None or indices is not None:
        return md.mla_decode_sparse(d.q, d.kv, d.block_table, d.seq_lens,
                                    d.indices if indices is None else indices, scale=w.scale,
                                    max_seq_len=w.max_seq_len, top_k=w.top_k,
                                    index_stride_b=w.index_stride_b, index_stride_q=w.index_stride_q,
                                    num_shards=w.num_shards, interleave=w.interleave,
                                    shard_id=-1 if shard_id is None else shard_id,
                                    out_dtype=out_dtype, workspace=workspace, stream=stream,
                                    kv_scale=d.kv_scale)
    if w.num_shards > 1:
        return md.mla_decode_dense(d.q, d.kv, d.block_table, d.seq_lens, scale=w.scale,
                                   max_seq_len=w.max_seq_len, num_shards=w.num_shards,
                                   interleave=w.interleave, shard_id=-1 if shard_id is None else shard_id,
                                   workspace=workspace, stream=stream, kv_scale=d.kv_scale)
    return md.mla_decode_dense(d.q, d.kv, d.block_table, d.seq_lens, scale=w.scale,
                               max_seq_len=w.max_seq_len, out_dtype=out_dtype, workspace=workspace,
                               stream=stream, kv_scale=d.kv_scale)
