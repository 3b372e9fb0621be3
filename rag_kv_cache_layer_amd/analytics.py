"""Deviation analytics on the GPU (CacheBlend sections 4.1-4.3, Figures 6-8).

Diagnostics around the fusor, run on the device with random weights:

* the attention deviation of a layer -- the L-2 norm of the difference
  between the forward attention matrix of the query rows under blending and
  under full prefill (section 4.1) -- as the recompute ratio grows (Figure 6);
* how concentrated the KV deviation is over the tokens of a layer (Figure 7);
* Spearman's rank correlation of the KV deviation between neighbouring
  layers (section 4.3, Figure 8).

Every step runs in the library: the layers (cb_full_prefill_layer,
cb_blend_layer), the query rows' Q (the Q those calls computed, read from
their workspace: cb_workspace_q_offset), the attention deviation
(cb_attention_deviation), ranks and correlation (cb_spearman) and the top
shares (cb_top_share).  torch holds the buffers; this module only sequences
the calls and copies results.
"""
from __future__ import annotations

import math
from typing import Dict, Sequence

from . import fusor as F


def _torch():
    import torch
    return torch


def precompute_chunks(cfg, layers, rope, x_all, offs, ws):
    """Each chunk prefilled alone through the stack at positions 0..L_c-1:
    per-layer K and V [T][n_kv][hd] in context order (keys at local
    positions; query rows left zero)."""
    torch = _torch()
    T = x_all.shape[0]
    L = len(layers)
    kv = (T, cfg.n_kv_heads, cfg.head_dim)
    dt = F.torch_dtype(cfg)
    K = torch.zeros((L,) + kv, dtype=dt, device=x_all.device)
    V = torch.zeros_like(K)
    for c in range(len(offs) - 1):
        lo, hi = int(offs[c]), int(offs[c + 1])
        x = x_all[lo:hi].contiguous()
        for l in range(L):
            y = torch.empty_like(x)
            F.full_prefill_layer(cfg, layers[l], rope, x, hi - lo, 0, K[l, lo:hi], V[l, lo:hi], y, ws)
            x = y
    return K, V


def full_stack(cfg, layers, rope, x_all, n_ctx, ws):
    """Full prefill through the stack: per-layer K, V and the Q of the query
    rows n_ctx .. T-1 as the library computed them."""
    torch = _torch()
    T = x_all.shape[0]
    kv = (T, cfg.n_kv_heads, cfg.head_dim)
    Ks, Vs, Qs = [], [], []
    x = x_all
    for layer in layers:
        k = torch.empty(kv, dtype=x.dtype, device=x.device)
        v = torch.empty_like(k)
        y = torch.empty_like(x)
        F.full_prefill_layer(cfg, layer, rope, x, T, 0, k, v, y, ws)
        Qs.append(F.workspace_q(cfg, ws, T, T)[n_ctx:].clone())
        Ks.append(k)
        Vs.append(v)
        x = y
    return Ks, Vs, Qs


def blend_stack(cfg, layers, rope, K, V, T, offs, x_first, ks, ws):
    """The fusor through the stack (re-alignment of every layer's keys, then
    gradual filtering, as fusor.blend_stack), keeping per layer the Q of the
    query rows and the deviations of the recomputed candidates."""
    torch = _torch()
    offs = [int(o) for o in offs]
    n_ctx, L0 = offs[-1], offs[1]
    q = T - n_ctx
    kv = cfg.n_kv_heads * cfg.head_dim
    F.rope_shift(cfg, rope, K, T * kv, len(layers), T, offs)
    dev_ = x_first.device
    s = torch.arange(L0, T, dtype=torch.int32, device=dev_)
    x = x_first
    Qs, devs = [], []
    for l, layer in enumerate(layers):
        m_in = s.numel()
        m_out = F.expected_m_out(T, n_ctx, m_in, ks[l])
        y = torch.empty((m_out, cfg.d_model), dtype=F.torch_dtype(cfg), device=dev_)
        so = torch.empty(m_out, dtype=torch.int32, device=dev_)
        dv = torch.empty(m_in, dtype=torch.float32, device=dev_)
        F.blend_layer(cfg, layer, rope, K[l], V[l], T, n_ctx, L0, s, m_in, x, None, ks[l], y, dv, so, ws)
        Qs.append(F.workspace_q(cfg, ws, T, m_in)[m_in - q:].clone())
        devs.append(dv[:m_in - q])
        s, x = so, y
    return Qs, devs


def stack_study(cfg, layers: Sequence[F.DeviceLayer], rope: F.DeviceRope, x_all, offs: Sequence[int],
                ratios_e4: Sequence[int], top_fracs=(0.1, 0.15, 0.2)) -> Dict[str, object]:
    """The three analyses on one stack and one input (x_all [T][d], the
    embeddings of the chunks in context order followed by the query).

    For each ratio r (units of 1e-4, the same k at every layer): the relative
    attention deviation ||A_l - A_l^full|| / ||A_l^full|| of the query rows
    per layer and its mean over layers.  From the r = 1 run (every candidate
    recomputed at every layer, so each deviation is the exact KV deviation):
    the share of the summed deviation in the top 10/15/20% of tokens per
    layer, and Spearman's correlation of the deviations of layers l, l+1 for
    l >= 1 (layer 0's inputs are the context-free embeddings, its deviation is
    rounding only)."""
    torch = _torch()
    T = x_all.shape[0]
    offs = [int(o) for o in offs]
    n_ctx, L0 = offs[-1], offs[1]
    n_cand = n_ctx - L0
    L = len(layers)
    ws = F.workspace(cfg, T, T, x_all.device)
    K0, V0 = precompute_chunks(cfg, layers, rope, x_all, offs, ws)
    Kf, Vf, Qf = full_stack(cfg, layers, rope, x_all, n_ctx, ws)
    last = torch.arange(n_ctx, T, dtype=torch.int32, device=x_all.device)
    out = {"ratios_e4": list(ratios_e4), "attn_dev": [], "attn_dev_mean": []}
    dev_r1 = None
    for r in ratios_e4:
        ks = F.filter_schedule(L, r, r, n_ctx, n_cand)
        K, V = K0.clone(), V0.clone()
        Qb, devs = blend_stack(cfg, layers, rope, K, V, T, offs, x_all[L0:].contiguous(), ks, ws)
        per = []
        for l in range(L):
            d2, n2 = F.attention_deviation(cfg, Qb[l], K[l], Qf[l], Kf[l], last)
            per.append(math.sqrt(d2 / n2))
        out["attn_dev"].append(per)
        out["attn_dev_mean"].append(sum(per) / L)
        if r >= 10000:
            dev_r1 = devs
    if dev_r1 is not None:
        out["top_share"] = {str(f): [F.top_share(d, int(math.ceil(f * d.numel() - 1e-9))) for d in dev_r1]
                            for f in top_fracs}
        out["spearman_neighbours"] = [F.spearman(dev_r1[l], dev_r1[l + 1]) for l in range(1, L - 1)]
    return out
