"""Deviation analytics on the GPU (CacheBlend sections 4.1-4.3, Figures 6-8).

Diagnostics around the fusor, run on the device with random weights:

* the attention deviation of a layer -- the L-2 norm of the difference
  between the forward attention matrix of the query rows under blending and
  under full prefill (section 4.1) -- as the recompute ratio grows (Figure 6);
* how concentrated the KV deviation is over the tokens of a layer (Figure 7);
* Spearman's rank correlation of the KV deviation between neighbouring
  layers (section 4.3, Figure 8).

The stacks run through the library (cb_full_prefill_layer, cb_blend_layer);
the statistics are small torch reductions on the results (fp32 attention
probabilities, fp64 sums).  The query rows' Q for the attention matrices is
projected here from each layer's stored input rows (RMSNorm, W_q, RoPE from
the library's own cos/sin tables), the same way for the blended and the
full-prefill run.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence

from . import fusor as F


def _torch():
    import torch
    return torch


def attention_matrix(q, k, last_key):
    """P [m][n_q][T] = softmax over t <= last_key[i] of q[i,h] . k[t, h // g] /
    sqrt(hd) (0 past last_key[i]); q [m][n_q][hd], k [T][n_kv][hd], fp32."""
    torch = _torch()
    m, n_q, hd = q.shape
    T, n_kv, _ = k.shape
    g = n_q // n_kv
    kt = k.float().permute(1, 2, 0).contiguous()                       # [n_kv][hd][T]
    s = torch.matmul(q.float().reshape(m, n_kv, g, hd), kt) / math.sqrt(hd)   # [m][n_kv][g][T]
    t = torch.arange(T, device=q.device)
    last = torch.as_tensor(last_key, device=q.device).reshape(m, 1, 1, 1)
    s = s.masked_fill(t.reshape(1, 1, 1, T) > last, float("-inf"))
    return torch.softmax(s, dim=-1).reshape(m, n_q, T)


def attention_deviation(a, b) -> float:
    """L-2 (Frobenius) norm of a - b."""
    d = (a.double() - b.double())
    return float(d.pow(2).sum().sqrt())


def ranks(x):
    """1-based ascending ranks; ties share the mean of the ranks they span."""
    torch = _torch()
    vals, inv, counts = torch.unique(x.double(), sorted=True, return_inverse=True, return_counts=True)
    ends = torch.cumsum(counts, 0).double()
    starts = ends - counts.double()
    return ((starts + 1.0 + ends) / 2.0)[inv]


def spearman(x, y) -> float:
    rx, ry = ranks(x), ranks(y)
    rx = rx - rx.mean()
    ry = ry - ry.mean()
    den = math.sqrt(float((rx * rx).sum()) * float((ry * ry).sum()))
    return float((rx * ry).sum()) / den if den > 0 else float("nan")


def top_share(dev, frac: float) -> float:
    """Share of the summed deviation held by the ceil(frac * n) largest."""
    torch = _torch()
    d = torch.sort(dev.double(), descending=True).values
    n = int(math.ceil(frac * d.numel() - 1e-9))
    tot = float(d.sum())
    return float(d[:n].sum()) / tot if tot > 0 else float("nan")


def query_q(cfg, layer: F.DeviceLayer, rope: F.DeviceRope, x, positions):
    """Q [m][n_q][hd] (fp32) of rows x [m][d] at the given positions:
    RMSNorm with the layer's gain, W_q, RoPE on interleaved pairs."""
    torch = _torch()
    xf = x.float()
    xn = xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + cfg.rms_eps) * layer.t["attn_norm"]
    q = torch.matmul(xn, layer.t["w_q"].float().t().contiguous()).reshape(x.shape[0], cfg.n_q_heads, cfg.head_dim)
    pos = torch.as_tensor(positions, device=x.device).long()
    c = rope.cos[pos].unsqueeze(1)   # [m][1][hd/2]
    s = rope.sin[pos].unsqueeze(1)
    a, b = q[..., 0::2], q[..., 1::2]
    out = torch.empty_like(q)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


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


def full_stack(cfg, layers, rope, x_all, ws):
    """Full prefill through the stack: per-layer K, V and each layer's input."""
    torch = _torch()
    T = x_all.shape[0]
    kv = (T, cfg.n_kv_heads, cfg.head_dim)
    Ks, Vs, xs = [], [], []
    x = x_all
    for layer in layers:
        k = torch.empty(kv, dtype=x.dtype, device=x.device)
        v = torch.empty_like(k)
        y = torch.empty_like(x)
        F.full_prefill_layer(cfg, layer, rope, x, T, 0, k, v, y, ws)
        Ks.append(k)
        Vs.append(v)
        xs.append(x)
        x = y
    return Ks, Vs, xs


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
    n_cand, q = n_ctx - L0, T - n_ctx
    L = len(layers)
    ws = F.workspace(cfg, T, T, x_all.device)
    K0, V0 = precompute_chunks(cfg, layers, rope, x_all, offs, ws)
    Kf, Vf, xf = full_stack(cfg, layers, rope, x_all, ws)
    qpos = list(range(n_ctx, T))
    A_full, A_norm = [], []
    for l in range(L):
        a = attention_matrix(query_q(cfg, layers[l], rope, xf[l][n_ctx:], qpos), Kf[l], qpos)
        A_full.append(a)
        A_norm.append(float(a.double().pow(2).sum().sqrt()))
    out = {"ratios_e4": list(ratios_e4), "attn_dev": [], "attn_dev_mean": []}
    dev_r1 = None
    for r in ratios_e4:
        ks = F.filter_schedule(L, r, r, n_ctx, n_cand)
        K, V = K0.clone(), V0.clone()
        res = F.blend_stack(cfg, layers, rope, K, V, T, offs, x_all[L0:].contiguous(), ks, ws)
        per = []
        for l in range(L):
            x_in = x_all[n_ctx:] if l == 0 else res[l - 1]["y"][-q:]
            a = attention_matrix(query_q(cfg, layers[l], rope, x_in, qpos), K[l], qpos)
            per.append(attention_deviation(a, A_full[l]) / A_norm[l])
        out["attn_dev"].append(per)
        out["attn_dev_mean"].append(sum(per) / L)
        if r >= 10000:
            dev_r1 = [res[l]["dev"][:n_cand].clone() for l in range(L)]
    if dev_r1 is not None:
        out["top_share"] = {str(f): [top_share(d, f) for d in dev_r1] for f in top_fracs}
        out["spearman_neighbours"] = [spearman(dev_r1[l], dev_r1[l + 1]) for l in range(1, L - 1)]
    return out
