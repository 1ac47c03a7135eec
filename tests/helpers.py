"""Shared helpers of the test suite: error metric, state comparison, device moves."""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import torch

# Tolerances on the maximum normwise relative error (float32 path / bf16 path).
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
# An output computed in float32 and rounded once to bfloat16 (7 stored mantissa
# bits, round to nearest) is off by at most 2^-8 of its own magnitude, hence by
# at most 2^-8 of the slice maximum.  Kernels whose arithmetic is all float32
# are held to that rounding floor plus the float32 bound.
TOL_BF16_ROUNDED = 2.0 ** -8 + TOL_F32


def has_gpu() -> bool:
    try:
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def f64(x) -> Optional[np.ndarray]:
    """Exact widening of a float32/bfloat16 tensor to a float64 numpy array."""
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def to_dev(d: Dict[str, Optional[torch.Tensor]], device="cuda") -> Dict[str, Optional[torch.Tensor]]:
    return {k: (None if v is None else v.to(device).contiguous()) for k, v in d.items()}


def slice_rel_err(x, r, lead: int = 2) -> float:
    """Max over the leading `lead` axes (e.g. (b, h)) of max|x - r| / max|r|."""
    x = f64(x)
    r = f64(r)
    assert x.shape == r.shape, (x.shape, r.shape)
    xs = x.reshape(int(np.prod(x.shape[:lead])), -1)
    rs = r.reshape(xs.shape)
    num = np.max(np.abs(xs - rs), axis=1)
    den = np.maximum(np.max(np.abs(rs), axis=1), 1e-30)
    if np.isnan(xs).any():
        return float("inf")
    return float(np.max(num / den))


def elem_rel_err(x, r, lead: int = 2) -> float:
    """Elementwise diagnostic beside the normwise error: max over the leading
    `lead` axes of max |x - r| / (|r| + 1e-3 max|r|).  It shows where single
    small elements are off, which the normwise figure hides; it is logged, not
    held to a tolerance."""
    x = f64(x)
    r = f64(r)
    assert x.shape == r.shape, (x.shape, r.shape)
    if np.isnan(x).any():
        return float("inf")
    xs = x.reshape(int(np.prod(x.shape[:lead])), -1)
    rs = r.reshape(xs.shape)
    floor = 1e-3 * np.max(np.abs(rs), axis=1, keepdims=True)
    den = np.maximum(np.abs(rs) + floor, 1e-300)
    return float(np.max(np.abs(xs - rs) / den))


def state_errors(C, n, m, Cr, nr, mr, lead: int = 2):
    """Errors of a final state against the oracle's.  The representation is
    unique only up to (C e^{-c}, n e^{-c}, m + c), so C and n are brought to the
    oracle's m first: x * exp(m - m_ref)."""
    C, n, m = f64(C), f64(n), f64(m)
    Cr, nr, mr = f64(Cr), f64(nr), f64(mr)
    scale = np.exp(m - mr)
    eC = slice_rel_err(C * scale[..., None, None], Cr, lead)
    en = slice_rel_err(n * scale[..., None], nr, lead)
    em = float(np.max(np.abs(m - mr)) / max(np.max(np.abs(mr)), 1e-30))
    return eC, en, em


def describe_err(name, e):
    return f"{name}: max normwise rel err {e:.3e}"


def sample_heads(B: int, H: int, count: int, seed: int = 0):
    """A fixed sample of (b, h) pairs that always includes the first and last head."""
    rng = np.random.default_rng(seed)
    allh = [(b, h) for b in range(B) for h in range(H)]
    if count >= len(allh):
        return allh
    pick = {0, len(allh) - 1}
    while len(pick) < count:
        pick.add(int(rng.integers(len(allh))))
    return [allh[i] for i in sorted(pick)]


def gather_heads(t: Optional[torch.Tensor], heads, dim_b=0, dim_h=1):
    """Stack the selected (b, h) slices of a [B,H,...] tensor into [1,N,...]."""
    if t is None:
        return None
    return torch.stack([t[b, h] for (b, h) in heads]).unsqueeze(0)


def finite(t: torch.Tensor) -> bool:
    return bool(torch.isfinite(t.float()).all().item())


def log(msg: str):
    print(msg, flush=True)


def nan_like(shape, dtype, device="cuda"):
    return torch.full(shape, math.nan, dtype=dtype, device=device)
