"""A plain Llama-style decoder layer for the oracle (test infrastructure only).

The fusor runs "the same attention module" as the model (CacheBlend paper,
section 4.2, the last step of the Figure 5b workflow) and its baseline is
"Full KV recompute" (section 7, baselines): the ordinary prefill of the whole
input.  The layer is the textbook Llama decoder without biases:

    xn = RMSNorm(x; g1)             x * g1 / sqrt(mean(x^2) + eps)
    Q, K, V = xn Wq^T, xn Wk^T, xn Wv^T
    Q, K    = RoPE at each row's absolute position
    O       = causal softmax(Q K^T / sqrt(hd)) V, query head h reads KV head
              h // (n_q / n_kv)  (grouped-query attention)
    h       = x + O Wo^T
    y       = h + W_down( silu(hn Wgate^T) * (hn Wup^T) ),  hn = RMSNorm(h; g2)

All arithmetic is in the dtype of the arrays given (fp32 by default).  With
``rowwise=True`` every projection is done one row at a time with a fixed
shape, so a row's result depends only on its own input and on the keys it
attends to; this is how the oracle reaches bit-exact prefix invariants.

``lin``, when given, replaces every projection: lin(x, name) returns x times
the weight called name (w_q, w_k, w_v, w_o, w_gate, w_up, w_down),
transposed; the 8-bit projections of oracle/fp8.py plug in here.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from .rope import apply_rope
from .storage import round_store  # noqa: F401  (re-exported)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    dt = x.dtype
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return (x / np.sqrt(ms + dt.type(eps))) * g.astype(dt)


def linear(x: np.ndarray, w: np.ndarray, rowwise: bool = False) -> np.ndarray:
    """x [m][in] times w^T (w in [out][in] layout)."""
    w = w.astype(x.dtype, copy=False)
    if not rowwise:
        return x @ w.T
    out = np.empty((x.shape[0], w.shape[0]), dtype=x.dtype)
    wt = np.ascontiguousarray(w.T)
    for i in range(x.shape[0]):
        out[i] = x[i:i + 1] @ wt
    return out


def silu(x: np.ndarray) -> np.ndarray:
    one = x.dtype.type(1.0)
    return x / (one + np.exp(-x))


def attention_rows(q: np.ndarray, k_all: np.ndarray, v_all: np.ndarray, last_key) -> np.ndarray:
    """Causal GQA attention of selected query rows over a key/value buffer.

    q [m][n_q][hd]; k_all, v_all [T][n_kv][hd]; query row i attends keys
    0 .. last_key[i] (inclusive).  Returns O [m][n_q][hd]."""
    m, n_q, hd = q.shape
    n_kv = k_all.shape[1]
    g = n_q // n_kv
    dt = q.dtype
    scale = dt.type(1.0 / math.sqrt(hd))
    kt = np.ascontiguousarray(k_all.transpose(1, 0, 2)).astype(dt, copy=False)  # [n_kv][T][hd]
    vt = np.ascontiguousarray(v_all.transpose(1, 0, 2)).astype(dt, copy=False)
    out = np.empty_like(q)
    for i in range(m):
        L = int(last_key[i]) + 1
        qi = q[i].reshape(n_kv, g, hd)                              # head h = n*g + j
        s = np.matmul(qi, kt[:, :L, :].transpose(0, 2, 1)) * scale  # [n_kv][g][L]
        s = s - s.max(axis=-1, keepdims=True)
        e = np.exp(s)
        p = e / e.sum(axis=-1, keepdims=True)
        out[i] = np.matmul(p, vt[:, :L, :]).reshape(n_q, hd)
    return out


def _proj(w, x, name, rowwise, lin):
    return linear(x, w[name], rowwise) if lin is None else lin(x, name)


def qkv_rows(w: Dict[str, np.ndarray], x: np.ndarray, positions, cfg, rowwise: bool = False, lin=None):
    """RMSNorm + Q/K/V projections + RoPE for rows at the given positions."""
    xn = rmsnorm(x, w["attn_norm"], cfg.rms_eps)
    n = x.shape[0]
    q = _proj(w, xn, "w_q", rowwise, lin).reshape(n, cfg.n_q_heads, cfg.head_dim)
    k = _proj(w, xn, "w_k", rowwise, lin).reshape(n, cfg.n_kv_heads, cfg.head_dim)
    v = _proj(w, xn, "w_v", rowwise, lin).reshape(n, cfg.n_kv_heads, cfg.head_dim)
    q = apply_rope(q, positions, cfg.rope_theta)
    k = apply_rope(k, positions, cfg.rope_theta)
    return q, k, v


def out_rows(w: Dict[str, np.ndarray], x: np.ndarray, o: np.ndarray, cfg, rowwise: bool = False,
             lin=None) -> np.ndarray:
    """Attention output projection, residual, RMSNorm, SwiGLU MLP, residual."""
    n = x.shape[0]
    h = x + _proj(w, o.reshape(n, -1), "w_o", rowwise, lin)
    hn = rmsnorm(h, w["mlp_norm"], cfg.rms_eps)
    u = silu(_proj(w, hn, "w_gate", rowwise, lin)) * _proj(w, hn, "w_up", rowwise, lin)
    return h + _proj(w, u, "w_down", rowwise, lin)


def full_prefill(w: Dict[str, np.ndarray], x: np.ndarray, cfg, pos0: int = 0,
                 rowwise: bool = False, store: Optional[str] = None, lin=None):
    """The ordinary layer over all rows of x at positions pos0 .. pos0+T-1.

    Returns (K [T][n_kv][hd], V, y [T][d]); K and V are rounded to the
    storage dtype before attention reads them (they are the stored cache)."""
    T = x.shape[0]
    pos = np.arange(pos0, pos0 + T)
    q, k, v = qkv_rows(w, x, pos, cfg, rowwise, lin)
    k = round_store(k, store)
    v = round_store(v, store)
    o = attention_rows(q, k, v, np.arange(T))
    y = out_rows(w, x, o, cfg, rowwise, lin)
    return k, v, round_store(y, store)
