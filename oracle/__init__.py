"""TEST INFRASTRUCTURE ONLY: the fp64 CPU reference for MLA decode attention.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never links, loads or
calls it, and it shares no code with the HIP path (the seeded input module
``latent_decode_attention_amd.workloads`` is the one thing both sides read).

The arithmetic is in ``mla_oracle.c`` (plain C, fp64, OpenMP over output rows);
this module compiles it with gcc and marshals numpy arrays through ctypes.
Functions return float64 arrays: ``out[n, d_v]`` and ``lse[n]`` for the selected
rows of the flattened ``[B, Q, h_q]`` output (all rows when ``rows`` is None).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile the oracle with gcc (IEEE fp64: no fast-math)."""
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(_Problem)
    i64p = ctypes.POINTER(ctypes.c_int64)
    dp = ctypes.POINTER(ctypes.c_double)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.oracle_dense.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                 i64p, dp, dp]
    lib.oracle_sparse.argtypes = [P, i32p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int64, i64p, dp, dp]
    lib.oracle_merge.argtypes = [dp, dp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, dp, dp]
    for f in (lib.oracle_dense, lib.oracle_sparse, lib.oracle_merge):
        f.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


class _Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Q", ctypes.c_int32), ("h_q", ctypes.c_int32),
                ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32), ("scale", ctypes.c_double),
                ("q", ctypes.c_void_p), ("kv", ctypes.c_void_p), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("max_blocks", ctypes.c_int32), ("seq_lens", ctypes.c_void_p),
                ("kv8", ctypes.c_void_p), ("kv_scale", ctypes.c_void_p)]


_ERRORS = {1: "bad argument", 2: "block table entry out of range", 3: "out of memory"}


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _problem(w, keep: list) -> _Problem:
    q = np.ascontiguousarray(w.q, dtype=np.uint16)
    kv = np.ascontiguousarray(w.kv, dtype=np.uint16)
    bt = np.ascontiguousarray(w.block_table, dtype=np.int32)
    sl = np.ascontiguousarray(w.seq_lens, dtype=np.int32)
    assert q.shape == (w.B, w.Q, w.h_q, w.d_qk)
    assert kv.ndim == 3 and kv.shape[2] == w.d_qk
    assert bt.ndim == 2 and bt.shape[0] == w.B and sl.shape == (w.B,)
    keep += [q, kv, bt, sl]
    kv8 = fac = None
    if getattr(w, "kv8", None) is not None:
        # The workload's cache is int8: the oracle reads the codes and factors.
        kv8 = np.ascontiguousarray(w.kv8, dtype=np.int8)
        fac = np.ascontiguousarray(w.kv_scale, dtype=np.float32)
        assert kv8.shape == kv.shape and fac.shape == kv.shape[:2]
        keep += [kv8, fac]
    return _Problem(w.B, w.Q, w.h_q, w.d_qk, w.d_v, float(w.scale), q.ctypes.data, kv.ctypes.data,
                    kv.shape[0], kv.shape[1], bt.ctypes.data, bt.shape[1], sl.ctypes.data,
                    None if kv8 is None else kv8.ctypes.data, None if fac is None else fac.ctypes.data)


def _sel(w, rows: Optional[Sequence[int]]):
    if rows is None:
        return None, w.B * w.Q * w.h_q
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    return r, r.size


def _check(rc: int):
    if rc != 0:
        raise RuntimeError("oracle failed: %s" % _ERRORS.get(rc, rc))


def dense(w, rows=None, num_shards: int = 1, interleave: int = 1, shard_id: int = 0):
    """Dense decode (optionally one DCP shard) for the selected output rows."""
    lib = _load()
    keep: list = []
    p = _problem(w, keep)
    sel, n = _sel(w, rows)
    out = np.zeros((n, w.d_v), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    rc = lib.oracle_dense(ctypes.byref(p), num_shards, interleave, shard_id, n,
                          None if sel is None else _ptr(sel, ctypes.c_int64),
                          _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    _check(rc)
    return out, lse


def sparse(w, rows=None, indices=None, top_k=None, stride_b=None, stride_q=None,
           num_shards: int = 1, interleave: int = 1, shard_id: int = 0):
    """Sparse (top-k) decode for the selected output rows (optionally one DCP shard:
    only the listed positions that shard holds)."""
    lib = _load()
    keep: list = []
    p = _problem(w, keep)
    idx = np.ascontiguousarray(w.indices if indices is None else indices, dtype=np.int32)
    top_k = w.top_k if top_k is None else top_k
    stride_b = w.index_stride_b if stride_b is None else stride_b
    stride_q = w.index_stride_q if stride_q is None else stride_q
    need = (w.B - 1) * stride_b + (w.Q - 1) * stride_q + top_k
    assert idx.size >= need, "index array smaller than its strides imply"
    sel, n = _sel(w, rows)
    out = np.zeros((n, w.d_v), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    rc = lib.oracle_sparse(ctypes.byref(p), _ptr(idx, ctypes.c_int32), top_k, stride_b, stride_q,
                           num_shards, interleave, shard_id, n,
                           None if sel is None else _ptr(sel, ctypes.c_int64),
                           _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double))
    _check(rc)
    return out, lse


def merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Online-softmax merge of partials o_parts[n, rows, d_v], lse_parts[n, rows]."""
    lib = _load()
    o = np.ascontiguousarray(o_parts, dtype=np.float64)
    l = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n, rows, d_v = o.shape
    assert l.shape == (n, rows)
    out = np.zeros((rows, d_v), dtype=np.float64)
    lse = np.zeros(rows, dtype=np.float64)
    _check(lib.oracle_merge(_ptr(o, ctypes.c_double), _ptr(l, ctypes.c_double), n, rows, d_v,
                            _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double)))
    return out, lse


def num_threads() -> int:
    return int(_load().oracle_num_threads())
