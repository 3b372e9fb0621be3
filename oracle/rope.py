"""Rotary position embedding for the oracle (test infrastructure only).

The CacheBlend paper (section 4.3, footnote 3) corrects a reused key's
position by multiplying each 2-D pair of the key by the rotation matrix
[[cos m*theta, -sin m*theta], [sin m*theta, cos m*theta]]; the aifetchly guide
("1. RoPE Delta Positional Realignment") states the composition
R(m + delta) = R(delta) R(m), so a key cached at local position m is moved to
m + delta by one more rotation by delta, and values are left alone.

Readings taken where the pages are silent:
* pairs are interleaved, (2i, 2i+1), with frequency theta_i = base^(-2i/hd)
  (the guide's simulator rotates the even / odd lanes of each head);
* tables are built in fp64 with the C library's pow / cos / sin (Python's
  ``math`` module) and rounded once to fp32; rotation arithmetic is done in
  the dtype of the data.
"""
from __future__ import annotations

import functools
import math

import numpy as np

from .storage import round_store


def inv_freq(theta: float, head_dim: int) -> list:
    """theta_i = base^(-2i/hd) in fp64, i = 0 .. hd/2 - 1."""
    return [math.pow(float(theta), -2.0 * i / head_dim) for i in range(head_dim // 2)]


@functools.lru_cache(maxsize=16)
def _table(theta: float, head_dim: int, n_pos: int):
    f = inv_freq(theta, head_dim)
    cos = np.empty((n_pos, head_dim // 2), dtype=np.float32)
    sin = np.empty((n_pos, head_dim // 2), dtype=np.float32)
    for p in range(n_pos):
        for i, fi in enumerate(f):
            a = float(p) * fi
            cos[p, i] = math.cos(a)
            sin[p, i] = math.sin(a)
    cos.setflags(write=False)
    sin.setflags(write=False)
    return cos, sin


def rope_table(theta: float, head_dim: int, positions) -> tuple:
    """(cos, sin), each fp32 [n][hd/2], for the given integer positions."""
    pos = np.asarray(positions, dtype=np.int64)
    if pos.size and int(pos.min()) < 0:
        raise ValueError("negative position")
    n_pos = int(pos.max()) + 1 if pos.size else 1
    cap = -(-n_pos // 4096) * 4096          # build tables in 4096-row steps
    cos, sin = _table(float(theta), int(head_dim), cap)
    return cos[pos], sin[pos]


def rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate interleaved pairs of x [n][H][hd] by per-row angles (cos/sin [n][hd/2]).

    (a, b) -> (a cos - b sin, a sin + b cos), computed in x's dtype."""
    dt = x.dtype
    c = cos.astype(dt)[:, None, :]
    s = sin.astype(dt)[:, None, :]
    a = x[..., 0::2]
    b = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def apply_rope(x: np.ndarray, positions, theta: float) -> np.ndarray:
    """RoPE of x [n][H][hd] at the given absolute positions."""
    cos, sin = rope_table(theta, x.shape[-1], positions)
    return rotate(x, cos, sin)


def rope_shift(k_cache: np.ndarray, chunk_offsets, theta: float, store=None) -> np.ndarray:
    """Re-rotate the cached keys of every chunk to its new absolute offset.

    k_cache [T][n_kv][hd] holds, for chunk c, keys rotated at local positions
    0 .. L_c-1 (precomputed in isolation).  Chunk c starts at row o_c, so its
    rows are rotated once more by delta = o_c.  Chunk 0 (delta = 0) and rows
    after the last chunk (the query) are returned unchanged.  The rotated rows
    are written back to the cache, so they are rounded to its storage dtype
    (``store``: None / 'f32' keep fp32, 'bf16' rounds to nearest even).
    Returns a new array; V needs no correction and is not an argument."""
    out = k_cache.copy()
    offs = [int(o) for o in chunk_offsets]
    for c in range(1, len(offs) - 1):
        lo, hi = offs[c], offs[c + 1]
        if hi <= lo:
            continue
        delta = np.full(hi - lo, lo, dtype=np.int64)
        cos, sin = rope_table(theta, k_cache.shape[-1], delta)
        out[lo:hi] = round_store(rotate(k_cache[lo:hi], cos, sin), store)
    return out
