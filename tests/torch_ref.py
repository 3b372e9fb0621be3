"""An independent PyTorch-CPU fp64 Llama decoder layer, used only to pin the
oracle.  It shares no code with ``oracle/``: RoPE is written as multiplication
by complex exponentials exp(i * p * theta_i) (angles in fp64, no fp32 table),
attention is ``torch.nn.functional.scaled_dot_product_attention`` with
``enable_gqa`` and RMSNorm / SwiGLU use torch primitives."""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def _t(a):
    return torch.as_tensor(np.asarray(a), dtype=torch.float64)


def rope_complex(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    """x [T][H][hd]; interleaved pairs as complex numbers."""
    T, H, hd = x.shape
    freqs = theta ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ang = pos.to(torch.float64)[:, None] * freqs[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)                 # [T][hd/2]
    xc = torch.view_as_complex(x.reshape(T, H, hd // 2, 2).contiguous())
    return torch.view_as_real(xc * rot[:, None, :]).reshape(T, H, hd)


def rms(x: torch.Tensor, g: torch.Tensor, eps: float) -> torch.Tensor:
    return x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + eps) * g


def layer(w, x, cfg, pos0: int = 0, attn_mask=None):
    """Returns (K [T][n_kv][hd], V, y [T][d]) in fp64 numpy."""
    x = _t(x)
    T = x.shape[0]
    nq, nkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    pos = torch.arange(pos0, pos0 + T)
    xn = rms(x, _t(w["attn_norm"]), cfg.rms_eps)
    q = (xn @ _t(w["w_q"]).T).reshape(T, nq, hd)
    k = (xn @ _t(w["w_k"]).T).reshape(T, nkv, hd)
    v = (xn @ _t(w["w_v"]).T).reshape(T, nkv, hd)
    q = rope_complex(q, pos, cfg.rope_theta)
    k = rope_complex(k, pos, cfg.rope_theta)
    if attn_mask is None:
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None].contiguous(),
                                           v.transpose(0, 1)[None].contiguous(), is_causal=True, enable_gqa=True)
    else:
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None].contiguous(),
                                           v.transpose(0, 1)[None].contiguous(), attn_mask=attn_mask, enable_gqa=True)
    o = o[0].transpose(0, 1).reshape(T, nq * hd)
    h = x + o @ _t(w["w_o"]).T
    hn = rms(h, _t(w["mlp_norm"]), cfg.rms_eps)
    y = h + (F.silu(hn @ _t(w["w_gate"]).T) * (hn @ _t(w["w_up"]).T)) @ _t(w["w_down"]).T
    return k.numpy(), v.numpy(), y.numpy()


def attention_masked(q, k, v, last_key):
    """Dense attention of q [m][nq][hd] over k, v [T][nkv][hd] with key t
    visible to query i iff t <= last_key[i]; via SDPA with a boolean mask."""
    q, k, v = _t(q), _t(k), _t(v)
    T = k.shape[0]
    mask = torch.arange(T)[None, :] <= torch.as_tensor(np.asarray(last_key))[:, None]
    o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None].contiguous(),
                                       v.transpose(0, 1)[None].contiguous(), attn_mask=mask, enable_gqa=True)
    return o[0].transpose(0, 1).numpy()


def rel_err(x, y) -> float:
    """max |x - y| / max |y| over the whole tensor."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    den = float(np.max(np.abs(y))) if y.size else 0.0
    return float(np.max(np.abs(x - y))) / den if den > 0 else float(np.max(np.abs(x - y), initial=0.0))
