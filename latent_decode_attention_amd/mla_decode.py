"""Python binding for libmla_decode (declared in include/mla_decode.h).

Argument marshalling only: torch tensors in, raw device pointers and the
current HIP stream out to the C ABI; every step of the computation runs in the
library's HIP kernels.  The functions carry the C entry points' names.  If the
library has not been built (``python -m latent_decode_attention_amd.build``)
importing this module raises, so nothing can silently fall back to another
implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_decode.so")

MLA_OK = 0
MLA_DTYPE_BF16 = 0
MLA_DTYPE_FP32 = 1
STATUS_NAMES = {0: "MLA_OK", 1: "MLA_ERR_NULL_POINTER", 2: "MLA_ERR_BAD_SHAPE",
                3: "MLA_ERR_UNSUPPORTED", 4: "MLA_ERR_WORKSPACE_TOO_SMALL", 5: "MLA_ERR_LAUNCH",
                6: "MLA_ERR_DEVICE", 7: "MLA_ERR_SCRATCH_LIMIT"}


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class Problem(ctypes.Structure):
    """Mirror of mla_problem_t."""
    _fields_ = [("B", ctypes.c_int32), ("Q", ctypes.c_int32), ("h_q", ctypes.c_int32),
                ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("scale", ctypes.c_float),
                ("q", ctypes.c_void_p), ("kv", ctypes.c_void_p), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("max_blocks", ctypes.c_int32), ("seq_lens", ctypes.c_void_p),
                ("max_seq_len", ctypes.c_int32), ("group_rows", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("kv_scale", ctypes.c_void_p)]


MLA_KV_BF16, MLA_KV_INT8 = 0, 1


class Plan(ctypes.Structure):
    """Mirror of mla_plan_t."""
    _fields_ = [("q_per_group", ctypes.c_int32), ("rows_per_group", ctypes.c_int32),
                ("units", ctypes.c_int32), ("splits", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("stream_len", ctypes.c_int32), ("grid", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmla_decode.so is not built; run `python -m latent_decode_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.mla_workspace_size.argtypes = [P, i32, i32, i32, i32, i64]
    lib.mla_workspace_size.restype = sz
    lib.mla_decode_dense.argtypes = [P, i32, i32, i32, vp, i32, vp, vp, sz, vp]
    lib.mla_decode_dense.restype = ctypes.c_int
    lib.mla_decode_sparse.argtypes = [P, vp, i32, i64, i64, vp, i32, vp, vp, sz, vp]
    lib.mla_decode_sparse.restype = ctypes.c_int
    lib.mla_merge_lse.argtypes = [vp, vp, i32, i64, i32, vp, i32, vp, vp]
    lib.mla_merge_lse.restype = ctypes.c_int
    lib.mla_kv_write.argtypes = [vp, vp, i64, vp, i64, vp, i32, i32, i32, vp]
    lib.mla_kv_write.restype = ctypes.c_int
    lib.mla_decode_sparse_noalloc.argtypes = [P, vp, i32, i64, i64, vp, i32, vp, vp]
    lib.mla_decode_sparse_noalloc.restype = ctypes.c_int
    lib.mla_decode_sparse_dcp.argtypes = [P, vp, i32, i64, i64, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.mla_decode_sparse_dcp.restype = ctypes.c_int
    lib.mla_topk_select.argtypes = [vp, i64, i64, vp, i32, i32, i32, i32, vp, vp]
    lib.mla_topk_select.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_plan_query.argtypes = [P, i32, i32, i32, i32, i64, i32, ctypes.POINTER(Plan)]
    lib.mla_plan_query.restype = ctypes.c_int
    return lib


lib = _load()


def mla_status_string(status: int) -> str:
    return lib.mla_status_string(int(status)).decode()


def _check(status: int):
    if status != MLA_OK:
        raise MlaError(status, mla_status_string(status))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(dtype) -> int:
    if dtype == torch.bfloat16:
        return MLA_DTYPE_BF16
    if dtype == torch.float32:
        return MLA_DTYPE_FP32
    raise TypeError("output dtype must be bfloat16 or float32")


# Work-group shape written into every problem this module builds (0: chosen
# per problem, or 64 / 128 query rows per work-group); tests set it to run
# each case under both shapes.
GROUP_ROWS = 0


def make_problem(q: torch.Tensor, kv: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                 scale: float, max_seq_len: int, kv_scale: Optional[torch.Tensor] = None) -> Problem:
    """mla_problem_t for q [B,Q,h_q,576] bf16, kv [N,bs,576] bf16 (or int8 with kv_scale fp32
    [N,bs], one factor per cache row), block_table [B,M] int32, seq_lens [B] int32."""
    kv_dt = torch.int8 if kv_scale is not None else torch.bfloat16
    checks = [("q", q, torch.bfloat16, 4), ("kv", kv, kv_dt, 3),
              ("block_table", block_table, torch.int32, 2), ("seq_lens", seq_lens, torch.int32, 1)]
    if kv_scale is not None:
        checks.append(("kv_scale", kv_scale, torch.float32, 2))
    for name, t, dt, nd in checks:
        if t.dtype != dt or t.dim() != nd or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous {nd}-d {dt} tensor")
        if not t.is_cuda:
            raise TypeError(f"{name} must live on the GPU")
    if kv_scale is not None and tuple(kv_scale.shape) != tuple(kv.shape[:2]):
        raise TypeError("kv_scale must be [num_blocks, block_size]")
    B, Q, h_q, d_qk = q.shape
    return Problem(B, Q, h_q, d_qk, 512, float(scale), q.data_ptr(), kv.data_ptr(), kv.shape[0],
                   kv.shape[1], block_table.data_ptr(), block_table.shape[1], seq_lens.data_ptr(),
                   int(max_seq_len), int(GROUP_ROWS), MLA_KV_BF16 if kv_scale is None else MLA_KV_INT8,
                   None if kv_scale is None else kv_scale.data_ptr())


def mla_workspace_size(problem: Problem, num_shards: int = 1, interleave: int = 1, shard_id: int = -1,
                       top_k: int = 0, index_stride_q: int = 0) -> int:
    n = lib.mla_workspace_size(ctypes.byref(problem), num_shards, interleave, shard_id, top_k, index_stride_q)
    if n == ctypes.c_size_t(-1).value:
        raise MlaError(2, "mla_workspace_size: invalid arguments")
    return int(n)


def mla_plan_query(problem: Problem, num_shards: int = 1, interleave: int = 1, shard_id: int = -1,
                   top_k: int = 0, index_stride_q: int = 0, num_cus: int = 256) -> dict:
    plan = Plan()
    _check(lib.mla_plan_query(ctypes.byref(problem), num_shards, interleave, shard_id, top_k,
                              index_stride_q, num_cus, ctypes.byref(plan)))
    return plan.as_dict()


def _workspace(problem, num_shards, interleave, shard_id, top_k, index_stride_q, workspace, device):
    need = mla_workspace_size(problem, num_shards, interleave, shard_id, top_k, index_stride_q)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace


def mla_decode_dense(q, kv, block_table, seq_lens, *, scale: float, max_seq_len: int,
                     num_shards: int = 1, interleave: int = 1, shard_id: int = -1,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     out_dtype=torch.bfloat16, workspace: Optional[torch.Tensor] = None, stream=None,
                     kv_scale: Optional[torch.Tensor] = None):
    """Dense decode (optionally DCP-sharded).  Returns (out, lse).  With kv_scale the
    cache is int8 and row r's values are kv_scale[r] * kv[r]."""
    p = make_problem(q, kv, block_table, seq_lens, scale, max_seq_len, kv_scale)
    B, Q, h_q, _ = q.shape
    sharded = num_shards > 1
    n_out = (num_shards if shard_id < 0 else 1) if sharded else 1
    if sharded:
        out_dtype = torch.float32
    oshape = (n_out, B, Q, h_q, 512) if sharded else (B, Q, h_q, 512)
    lshape = (n_out, B, Q, h_q) if sharded else (B, Q, h_q)
    if out is None:
        out = torch.empty(oshape, dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty(lshape, dtype=torch.float32, device=q.device)
    if tuple(out.shape) != oshape or tuple(lse.shape) != lshape or lse.dtype != torch.float32:
        raise TypeError("out/lse have the wrong shape or dtype")
    workspace = _workspace(p, num_shards, interleave, shard_id, 0, 0, workspace, q.device)
    _check(lib.mla_decode_dense(ctypes.byref(p), num_shards, interleave, shard_id, _ptr(out),
                                _dtype_code(out.dtype), _ptr(lse), _ptr(workspace),
                                0 if workspace is None else workspace.numel(), _stream(stream)))
    return out, lse


def mla_decode_sparse(q, kv, block_table, seq_lens, indices, *, scale: float, max_seq_len: int,
                      top_k: Optional[int] = None, index_stride_b: Optional[int] = None,
                      index_stride_q: Optional[int] = None, num_shards: int = 1, interleave: int = 1,
                      shard_id: int = -1, out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
                      workspace: Optional[torch.Tensor] = None, stream=None,
                      kv_scale: Optional[torch.Tensor] = None):
    """Sparse top-k decode.  indices: int32, [B, top_k] (shared across Q) or [B, Q, top_k].
    With num_shards > 1 (mla_decode_sparse_dcp) each DCP shard attends the listed
    positions it holds and emits fp32 partials [n_out, B, Q, h_q, 512] and lse.  With
    kv_scale the cache is int8 (as in mla_decode_dense)."""
    p = make_problem(q, kv, block_table, seq_lens, scale, max_seq_len, kv_scale)
    if indices.dtype != torch.int32 or not indices.is_contiguous() or not indices.is_cuda:
        raise TypeError("indices must be a contiguous int32 GPU tensor")
    B, Q, h_q, _ = q.shape
    if top_k is None:
        top_k = indices.shape[-1]
    if index_stride_q is None:
        index_stride_q = top_k if indices.dim() == 3 else 0
    if index_stride_b is None:
        index_stride_b = (indices.shape[1] * top_k) if indices.dim() == 3 else top_k
    need = (B - 1) * index_stride_b + (Q - 1) * index_stride_q + top_k
    if indices.numel() < need:
        raise TypeError("indices is smaller than its strides imply")
    if num_shards > 1:
        n_out = num_shards if shard_id < 0 else 1
        if out is None:
            out = torch.empty((n_out, B, Q, h_q, 512), dtype=torch.float32, device=q.device)
        if lse is None:
            lse = torch.empty((n_out, B, Q, h_q), dtype=torch.float32, device=q.device)
        if (tuple(out.shape) != (n_out, B, Q, h_q, 512) or out.dtype != torch.float32 or
                tuple(lse.shape) != (n_out, B, Q, h_q) or lse.dtype != torch.float32):
            raise TypeError("sharded out/lse must be fp32 [n_out, B, Q, h_q, 512] and [n_out, B, Q, h_q]")
        workspace = _workspace(p, num_shards, interleave, shard_id, top_k, index_stride_q, workspace, q.device)
        _check(lib.mla_decode_sparse_dcp(ctypes.byref(p), _ptr(indices), top_k, index_stride_b,
                                         index_stride_q, num_shards, interleave, shard_id, _ptr(out),
                                         _ptr(lse), _ptr(workspace),
                                         0 if workspace is None else workspace.numel(), _stream(stream)))
        return out, lse
    if out is None:
        out = torch.empty((B, Q, h_q, 512), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Q, h_q), dtype=torch.float32, device=q.device)
    workspace = _workspace(p, 1, 1, -1, top_k, index_stride_q, workspace, q.device)
    _check(lib.mla_decode_sparse(ctypes.byref(p), _ptr(indices), top_k, index_stride_b, index_stride_q,
                                 _ptr(out), _dtype_code(out.dtype), _ptr(lse), _ptr(workspace),
                                 0 if workspace is None else workspace.numel(), _stream(stream)))
    return out, lse


def mla_decode_sparse_noalloc(q, kv, block_table, seq_lens, indices, *, scale: float, max_seq_len: int,
                              top_k: Optional[int] = None, index_stride_b: Optional[int] = None,
                              index_stride_q: Optional[int] = None, out: torch.Tensor, lse: torch.Tensor,
                              stream=None, kv_scale: Optional[torch.Tensor] = None):
    """mla_decode_sparse into caller-given out [B,Q,h_q,512] (bf16 or fp32) and lse [B,Q,h_q]
    fp32, with the library's fixed device scratch instead of a workspace: allocates nothing."""
    p = make_problem(q, kv, block_table, seq_lens, scale, max_seq_len, kv_scale)
    if indices.dtype != torch.int32 or not indices.is_contiguous() or not indices.is_cuda:
        raise TypeError("indices must be a contiguous int32 GPU tensor")
    B, Q, h_q, _ = q.shape
    if top_k is None:
        top_k = indices.shape[-1]
    if index_stride_q is None:
        index_stride_q = top_k if indices.dim() == 3 else 0
    if index_stride_b is None:
        index_stride_b = (indices.shape[1] * top_k) if indices.dim() == 3 else top_k
    if indices.numel() < (B - 1) * index_stride_b + (Q - 1) * index_stride_q + top_k:
        raise TypeError("indices is smaller than its strides imply")
    if tuple(out.shape) != (B, Q, h_q, 512) or tuple(lse.shape) != (B, Q, h_q) or lse.dtype != torch.float32:
        raise TypeError("out/lse have the wrong shape or dtype")
    _check(lib.mla_decode_sparse_noalloc(ctypes.byref(p), _ptr(indices), top_k, index_stride_b, index_stride_q,
                                         _ptr(out), _dtype_code(out.dtype), _ptr(lse), _stream(stream)))
    return out, lse


def mla_merge_lse(o_parts: torch.Tensor, lse_parts: torch.Tensor, *, out: Optional[torch.Tensor] = None,
                  lse_out: Optional[torch.Tensor] = None, out_dtype=torch.float32, stream=None):
    """Merge partials o_parts [n, ..., d_v] fp32 with lse_parts [n, ...] fp32."""
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("partials must be float32")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous() and o_parts.is_cuda):
        raise TypeError("partials must be contiguous GPU tensors")
    n, d_v = o_parts.shape[0], o_parts.shape[-1]
    rows = o_parts.numel() // (n * d_v)
    if lse_parts.numel() != n * rows:
        raise TypeError("lse_parts does not match o_parts")
    if out is None:
        out = torch.empty(o_parts.shape[1:], dtype=out_dtype, device=o_parts.device)
    if lse_out is None:
        lse_out = torch.empty(lse_parts.shape[1:], dtype=torch.float32, device=o_parts.device)
    _check(lib.mla_merge_lse(_ptr(o_parts), _ptr(lse_parts), n, rows, d_v, _ptr(out),
                             _dtype_code(out.dtype), _ptr(lse_out), _stream(stream)))
    return out, lse_out


def mla_kv_write(rows: torch.Tensor, slot_mapping: torch.Tensor, kv: torch.Tensor, *,
                 positions: Optional[torch.Tensor] = None, num_shards: int = 1, interleave: int = 1,
                 shard_id: int = 0, stream=None) -> torch.Tensor:
    """Store rows [T, 576] bf16 into the paged cache kv [num_blocks, block_size, 576] bf16
    at slot_mapping [T] int32 (negative: not stored); with num_shards > 1 only the
    tokens whose positions [T] int32 this shard owns.  Updates kv in place."""
    if rows.dtype != torch.bfloat16 or kv.dtype != torch.bfloat16:
        raise TypeError("rows and kv must be bfloat16")
    if slot_mapping.dtype != torch.int32 or (positions is not None and positions.dtype != torch.int32):
        raise TypeError("slot_mapping and positions must be int32")
    for name, t in (("rows", rows), ("slot_mapping", slot_mapping), ("kv", kv), ("positions", positions)):
        if t is not None and (not t.is_contiguous() or not t.is_cuda):
            raise TypeError(f"{name} must be a contiguous GPU tensor")
    T = rows.shape[0] if rows.dim() == 2 else 0
    if rows.dim() != 2 or rows.shape[1] != 576 or slot_mapping.numel() != T or kv.shape[-1] != 576:
        raise TypeError("expected rows [T, 576], slot_mapping [T], kv [..., 576]")
    if positions is not None and positions.numel() != T:
        raise TypeError("positions must have one entry per row")
    _check(lib.mla_kv_write(_ptr(rows), _ptr(slot_mapping), T, _ptr(kv), kv.numel() // 576, _ptr(positions),
                            num_shards, interleave, shard_id, _stream(stream)))
    return kv


def mla_topk_select(scores: torch.Tensor, seq_lens: torch.Tensor, top_k: int, *,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Top-k positions of indexer scores [B, Q, max_len] fp32 (rows stop at the causal
    limit seq_lens[b] - Q + q + 1): int32 [B, Q, top_k], ascending, -1 padded."""
    if scores.dtype != torch.float32 or scores.dim() != 3 or not scores.is_cuda or scores.stride(2) != 1:
        raise TypeError("scores must be a float32 GPU tensor [B, Q, max_len] with unit last stride")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous() or not seq_lens.is_cuda:
        raise TypeError("seq_lens must be a contiguous int32 GPU tensor")
    B, Q, max_len = scores.shape
    if seq_lens.numel() != B:
        raise TypeError("seq_lens must have B entries")
    if out is None:
        out = torch.empty((B, Q, top_k), dtype=torch.int32, device=scores.device)
    if out.dtype != torch.int32 or tuple(out.shape) != (B, Q, top_k) or not out.is_contiguous():
        raise TypeError("out must be a contiguous int32 tensor [B, Q, top_k]")
    _check(lib.mla_topk_select(_ptr(scores), scores.stride(0), scores.stride(1), _ptr(seq_lens), B, Q, max_len,
                               top_k, _ptr(out), _stream(stream)))
    return out
