"""Rounding of values written to stored tensors (test infrastructure only).

KV caches and layer outputs are stored tensors: when the workload stores them
in bf16, every value written is rounded to bf16 (round to nearest even) before
anything reads it back.
"""
from __future__ import annotations

import numpy as np


def round_store(x: np.ndarray, store) -> np.ndarray:
    """Round to the storage dtype ('f32', 'f64' or None = no rounding, 'bf16' = RNE)."""
    if store in ("f32", "f64", None):
        return x
    if store != "bf16":
        raise ValueError(store)
    dt = x.dtype
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(dt)
