"""Inputs of a single fusor layer whose deviations come from missing
cross-attention (test infrastructure only).

A single decoder layer fed the same hidden states for the isolated precompute
and for the blended call would see K deviations made of rounding alone: the
difference the CacheBlend paper ranks tokens by (section 4.1, KV deviation;
section 3.3, the missing cross-attention between chunks) only appears once a
layer below has mixed context.  The single-layer workloads therefore model the
measured layer as the second layer of a two-layer stack whose two layers share
one set of weights W:

* isolated: H_iso[c] = Layer_W(E_c) at positions 0 .. L_c-1 for each chunk
  alone; K_pre[c], V_pre[c] = the QKV projections of H_iso[c] at the same
  local positions (keys rotated at local positions);
* full:     H_full   = Layer_W(E_all) over the whole input at positions 0 .. T-1.

The measured call receives K_pre / V_pre (in context order, then shifted) as
its cache and rows of H_full as its hidden inputs.  This is exactly layer 1 of
the stack driver with layers [W, W].
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .layer import full_prefill, qkv_rows, round_store


def single_layer_inputs(w: Dict[str, np.ndarray], cfg, e_chunks: Sequence[np.ndarray], e_query: np.ndarray,
                        rowwise: bool = False, store: Optional[str] = None) -> Dict[str, np.ndarray]:
    """e_chunks: chunk embeddings in context order.  Returns
    k_pre, v_pre [T][n_kv][hd] (query rows zero), hidden [T][d] = H_full,
    offsets [n_chunks+1]."""
    lens = [e.shape[0] for e in e_chunks]
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n_ctx = int(offsets[-1])
    T = n_ctx + e_query.shape[0]
    dt = e_query.dtype
    k_pre = np.zeros((T, cfg.n_kv_heads, cfg.head_dim), dtype=dt)
    v_pre = np.zeros((T, cfg.n_kv_heads, cfg.head_dim), dtype=dt)
    for c, e in enumerate(e_chunks):
        _, _, h_iso = full_prefill(w, e, cfg, 0, rowwise, store)
        _, k, v = qkv_rows(w, h_iso, np.arange(e.shape[0]), cfg, rowwise)
        lo, hi = int(offsets[c]), int(offsets[c + 1])
        k_pre[lo:hi] = round_store(k, store)
        v_pre[lo:hi] = round_store(v, store)
    e_all = np.concatenate(list(e_chunks) + [e_query], axis=0)
    _, _, h_full = full_prefill(w, e_all, cfg, 0, rowwise, store)
    return {"k_pre": k_pre, "v_pre": v_pre, "hidden": h_full, "offsets": offsets}
