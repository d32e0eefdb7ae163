"""Parity bars shared by the GPU tests, and a record of the errors they saw.

The bars (the parity contract: max-abs error <= 1e-2 on O computed with fp32
accumulation and stored as bf16, <= 1e-3 on lse; with the reading for bf16
outputs of large magnitude):
  * lse: |Δ| <= 1e-3 everywhere (both -inf counts as equal);
  * O stored as fp32: |Δ| <= 1e-2 everywhere;
  * O stored as bf16: |Δ| <= 1e-2 where |O_ref| < 4, and <= 1 bf16 ulp of O_ref
    where |O_ref| >= 4.  Rounding to bf16 alone moves a value by up to half an
    ulp, which is more than 1e-2 once |O| >= 4 (an ulp there is >= 2^-5), so the
    literal bound cannot apply there; below 4 it does, unchanged.

Every comparison is recorded (largest |ΔO|, |Δlse| and |O_ref| per label), and
conftest writes the record to the JSON file named by MLA_PARITY_REPORT at the
end of the session.
"""
from __future__ import annotations

import numpy as np

O_ABS_TOL = 1e-2
LSE_ABS_TOL = 1e-3
BF16_ABS_LIMIT = 4.0  # below this |O_ref|, bf16 outputs keep the absolute bound

RECORD: dict = {}


def ulp_bf16(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def o_tolerance(o_ref, bf16_out: bool):
    o_ref = np.asarray(o_ref, dtype=np.float64)
    if not bf16_out:
        return np.full_like(o_ref, O_ABS_TOL)
    return np.where(np.abs(o_ref) < BF16_ABS_LIMIT, O_ABS_TOL, ulp_bf16(o_ref))


def _note(label, **kw):
    if not label:
        return
    r = RECORD.setdefault(label, {})
    for k, v in kw.items():
        if v is None:
            continue
        if k.startswith("max_"):
            r[k] = max(r.get(k, 0.0), float(v))
        else:
            r[k] = v


def check_o(o_gpu, o_ref, what="", bf16_out=None, label=None):
    """Element-wise O bar.  o_gpu: a torch tensor (bf16 or fp32) or numpy array."""
    try:
        import torch
        is_tensor = isinstance(o_gpu, torch.Tensor)
    except ImportError:  # pragma: no cover
        is_tensor = False
    if is_tensor:
        if bf16_out is None:
            bf16_out = o_gpu.dtype == torch.bfloat16
        g = o_gpu.float().cpu().numpy().astype(np.float64)
    else:
        g = np.asarray(o_gpu, dtype=np.float64)
        bf16_out = bool(bf16_out)
    g = g.reshape(o_ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - o_ref)
    tol = o_tolerance(o_ref, bf16_out)
    bad = err > tol
    small = np.abs(o_ref) < BF16_ABS_LIMIT
    _note(label, max_abs_dO=err.max() if err.size else 0.0,
          max_abs_dO_below_4=(err[small].max() if small.any() else 0.0),
          max_abs_O_ref=np.abs(o_ref).max() if o_ref.size else 0.0,
          out_dtype="bf16" if bf16_out else "fp32", rows=int(o_ref.size // o_ref.shape[-1]) if o_ref.size else 0)
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance, max err {err.max():.3g} "
                           f"(worst excess {float((err - tol).max()):.3g} at |O_ref| = "
                           f"{float(np.abs(o_ref).reshape(-1)[np.argmax((err - tol).reshape(-1))]):.3g})")
    return float(err.max()) if err.size else 0.0


def check_lse(l_gpu, l_ref, what="", label=None):
    try:
        import torch
        if isinstance(l_gpu, torch.Tensor):
            l_gpu = l_gpu.float().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    g = np.asarray(l_gpu, dtype=np.float64).reshape(l_ref.shape)
    both_inf = np.isneginf(g) & np.isneginf(l_ref)
    err = np.where(both_inf, 0.0, np.abs(g - l_ref))
    _note(label, max_abs_dlse=np.nanmax(err) if err.size else 0.0)
    assert np.all(err <= LSE_ABS_TOL), f"{what}: lse max err {np.nanmax(err):.3g}"
    return float(err.max()) if err.size else 0.0
