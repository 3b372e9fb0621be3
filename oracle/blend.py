"""The CacheBlend fusor, step by step, for the oracle (test infrastructure only).

Sources (CacheBlend paper, arXiv 2405.16444):
* section 4.1, Table 1: KV deviation of token j on layer i, the difference
  between the reused KV and the fully recomputed KV of that token;
* section 4.2, Figure 5b: one layer of selective recompute -- mask the layer
  input down to the selected tokens, compute their Q/K/V, expand K/V with the
  reused entries of the other tokens, run attention to produce the next
  layer's input;  compute is proportional to the number of selected tokens;
* section 4.3: pick the tokens with the highest KV deviation (HKVD); prefill
  the first layer fully, then filter gradually -- the tokens recomputed on a
  layer are ranked by their deviation there and the top ones are recomputed
  on the next layer (Figure 9); the reused keys are re-rotated to their new
  positions (footnote 3).
The ml-canon note "54 Prefix Caching -> CacheBlend" sketches the same
loop (deviation, top-k of r*len, recompute layer by layer).

Readings taken where the pages are silent or disagree (each also listed in
the design notes of the repository):
* deviation = squared L2 norm of (new K row - cached K row) over all KV heads,
  computed from stored values before the cache row is overwritten;
* ranking is by deviation descending, ties broken by the lower token index;
  the kept set is returned in ascending token order;
* the token count of a ratio r is ceil(r * n_ctx), capped at the candidate
  count, computed exactly from r in units of 1e-4;
* the first chunk is the prefix: it is never recomputed nor re-rotated; query
  rows are new tokens, always recomputed, never ranked;
* on the layer that selects, every recomputed row keeps its new K/V; only
  the kept rows continue through attention and the MLP;
* layer 0 recomputes all candidates without selecting, layer 1 recomputes
  them again and selects; gradual filtering lowers the ratio linearly from
  r_first at layer 1 to r_last at the last layer, never growing the set.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Dict, List, Optional, Sequence

import numpy as np

from .layer import attention_rows, full_prefill, out_rows, qkv_rows, round_store
from .rope import rope_shift


# --------------------------------------------------------------------------
# counts and selection
# --------------------------------------------------------------------------

def num_selected(r_e4: int, n_ctx: int, n_cand: int) -> int:
    """HKVD count for ratio r = r_e4 / 1e4: min(ceil(r * n_ctx), n_cand), exact."""
    if r_e4 < 0 or n_ctx < 0 or n_cand < 0:
        raise ValueError("negative argument")
    k = math.ceil(Fraction(r_e4 * n_ctx, 10000))
    return int(min(k, n_cand))


def filter_schedule(n_layers: int, r_first_e4: int, r_last_e4: int, n_ctx: int, n_cand: int) -> List[int]:
    """Per-layer k_out.  Layer 0 keeps every candidate (no selection).  Layer
    l >= 1 keeps k_l = ceil(r_l * n_ctx) with r_l falling linearly from
    r_first (l = 1) to r_last (l = L-1); r_last_e4 == 0 means a constant ratio.
    k never grows from one layer to the next."""
    ks = [n_cand]
    for l in range(1, n_layers):
        if r_last_e4 == 0 or n_layers <= 2:
            r = Fraction(r_first_e4)
        else:
            r = Fraction(r_first_e4) - Fraction(r_first_e4 - r_last_e4) * Fraction(l - 1, n_layers - 2)
        k = math.ceil(r * n_ctx / 10000)
        ks.append(int(min(k, n_cand, ks[-1])))
    return ks


def topk_hkvd(dev: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest deviations, ranked by (deviation descending,
    index ascending), returned in ascending index order."""
    n = len(dev)
    k = max(0, min(int(k), n))
    order = sorted(range(n), key=lambda i: (-float(dev[i]), i))
    return np.array(sorted(order[:k]), dtype=np.int64)


def k_deviation(k_new: np.ndarray, k_old: np.ndarray) -> np.ndarray:
    """Per-token squared L2 deviation over all KV heads: [n][n_kv][hd] -> [n]."""
    n = k_new.shape[0]
    d = (k_new - k_old).reshape(n, int(np.prod(k_new.shape[1:])))
    return np.sum(d * d, axis=1)


# --------------------------------------------------------------------------
# one fusor layer
# --------------------------------------------------------------------------

def blend_layer(w: Dict[str, np.ndarray], cfg, k_cache: np.ndarray, v_cache: np.ndarray,
                n_ctx: int, s_in: np.ndarray, x_in: np.ndarray, k_out: int,
                rowwise: bool = False, store: Optional[str] = None,
                keep: Optional[np.ndarray] = None, lin=None) -> Dict[str, np.ndarray]:
    """One layer of selective recompute.

    k_cache, v_cache [T][n_kv][hd]: this layer's cache (keys already moved to
    their absolute positions); copies are returned, the inputs are untouched.
    s_in: ascending token rows to recompute; they are candidate rows (< n_ctx)
    followed by every query row (>= n_ctx).  x_in[i] is the layer input of row
    s_in[i].  k_out: how many candidate rows to keep for attention, the MLP
    and the next layer.

    Returns k_cache, v_cache (new K/V written for every row of s_in), dev
    [m_in] (NaN on query rows), sel (positions into s_in), s_out = s_in[sel]
    and y [m_out][d], the layer output of the kept rows in s_out order.

    keep: optional teacher forcing of step 4 -- ascending positions into s_in
    of the candidate rows to keep instead of the top-k by deviation (used to
    compare another implementation on the same selection).  lin: the
    projections, as in oracle.layer (None = fp32 products with w)."""
    s_in = np.asarray(s_in, dtype=np.int64)
    T = k_cache.shape[0]
    if np.any(np.diff(s_in) <= 0):
        raise ValueError("s_in must be strictly ascending")
    if not np.array_equal(s_in[s_in >= n_ctx], np.arange(n_ctx, T)):
        raise ValueError("s_in must hold every query row")
    # 1. Q/K/V of the selected rows only (Figure 5b: mask, then project)
    q, k, v = qkv_rows(w, x_in, s_in, cfg, rowwise, lin)
    k = round_store(k, store)
    v = round_store(v, store)
    # 2. deviation against the reused entry, before it is replaced
    cand = np.nonzero(s_in < n_ctx)[0]
    dev = np.full(len(s_in), np.nan, dtype=x_in.dtype)
    dev[cand] = k_deviation(k[cand], k_cache[s_in[cand]].astype(k.dtype))
    # 3. expand: reused rows stay, recomputed rows get their new K/V
    kc = k_cache.copy()
    vc = v_cache.copy()
    kc[s_in] = k
    vc[s_in] = v
    # 4. keep the HKVD rows plus the query rows
    if keep is None:
        keep = cand[topk_hkvd(dev[cand], min(k_out, len(cand)))]
    else:
        keep = np.asarray(keep, dtype=np.int64)
        if not np.all(np.isin(keep, cand)) or np.any(np.diff(keep) <= 0):
            raise ValueError("keep must be ascending candidate positions")
    sel = np.concatenate([keep, np.nonzero(s_in >= n_ctx)[0]])
    s_out = s_in[sel]
    # 5. attention of the kept rows over the blended cache, causal
    o = attention_rows(q[sel], kc.astype(q.dtype), vc.astype(q.dtype), s_out)
    # 6. rest of the layer for the kept rows
    y = round_store(out_rows(w, x_in[sel], o, cfg, rowwise, lin), store)
    return {"k_cache": kc, "v_cache": vc, "dev": dev, "sel": sel, "s_out": s_out, "y": y}


# --------------------------------------------------------------------------
# stacks
# --------------------------------------------------------------------------

def precompute_chunk(ws: Sequence[Dict[str, np.ndarray]], cfg, e_chunk: np.ndarray,
                     rowwise: bool = False, store: Optional[str] = None):
    """Prefill one chunk alone at positions 0 .. L-1 through every layer and
    keep its K/V per layer (the isolated precompute, KV^pre)."""
    ks, vs = [], []
    x = e_chunk
    for w in ws:
        k, v, x = full_prefill(w, x, cfg, 0, rowwise, store)
        ks.append(k)
        vs.append(v)
    return ks, vs


def assemble_caches(cfg, chunk_kv: Dict[int, tuple], order: Sequence[int], T: int, n_layers: int, dtype=np.float32):
    """Per-layer caches [T][n_kv][hd] with the chunks' K/V in context order;
    query rows start at zero (they are always recomputed before being read)."""
    K = [np.zeros((T, cfg.n_kv_heads, cfg.head_dim), dtype=dtype) for _ in range(n_layers)]
    V = [np.zeros((T, cfg.n_kv_heads, cfg.head_dim), dtype=dtype) for _ in range(n_layers)]
    row = 0
    for c in order:
        ks, vs = chunk_kv[c]
        L = ks[0].shape[0]
        for l in range(n_layers):
            K[l][row:row + L] = ks[l]
            V[l][row:row + L] = vs[l]
        row += L
    return K, V


def shift_caches(cfg, K: Sequence[np.ndarray], offsets, store: Optional[str] = None) -> List[np.ndarray]:
    return [rope_shift(k, offsets, cfg.rope_theta, store) for k in K]


def blend_stack(ws: Sequence[Dict[str, np.ndarray]], cfg, K: Sequence[np.ndarray], V: Sequence[np.ndarray],
                n_ctx: int, first_chunk_len: int, x_all: np.ndarray, ks: Sequence[int],
                rowwise: bool = False, store: Optional[str] = None) -> Dict[str, list]:
    """Run the fusor through every layer.

    K, V: per-layer caches after the position shift.  x_all [T][d]: the input
    embeddings of all rows.  ks: per-layer k_out (filter_schedule).  Layer 0
    starts from every candidate row plus the query rows."""
    T = x_all.shape[0]
    s = np.concatenate([np.arange(first_chunk_len, n_ctx), np.arange(n_ctx, T)])
    x = x_all[s]
    out = {"K": [], "V": [], "S": [], "dev": [], "y": None, "s_last": None}
    for l, w in enumerate(ws):
        r = blend_layer(w, cfg, K[l], V[l], n_ctx, s, x, ks[l], rowwise, store)
        out["K"].append(r["k_cache"])
        out["V"].append(r["v_cache"])
        out["S"].append(s)
        out["dev"].append(r["dev"])
        s, x = r["s_out"], r["y"]
    out["y"], out["s_last"] = x, s
    return out


def full_prefill_stack(ws: Sequence[Dict[str, np.ndarray]], cfg, x_all: np.ndarray,
                       rowwise: bool = False, store: Optional[str] = None):
    """Full KV recompute through every layer: per-layer K, V and the output."""
    Ks, Vs = [], []
    x = x_all
    for w in ws:
        k, v, x = full_prefill(w, x, cfg, 0, rowwise, store)
        Ks.append(k)
        Vs.append(v)
    return Ks, Vs, x
