"""MLA decode attention over a paged latent KV cache, hand-written HIP for gfx950.

The compute path lives in the C-ABI library ``libmla_decode.so`` (declared in
``include/mla_decode.h``); :mod:`latent_decode_attention_amd.mla_decode` is a thin
ctypes binding over it.  Importing this package loads nothing; the binding loads
the library on first use and raises if it is missing.
"""
__all__ = ["mla_decode", "workloads"]
