"""Deviation analytics of the oracle (test infrastructure only).

CacheBlend (arXiv 2405.16444) section 4.1 defines, per layer i, the KV
deviation of token j (how far its reused KV is from the fully recomputed one)
and the attention deviation: the L-2 norm of the difference between the
layer's forward attention matrix and the one of full prefill.  Section 4.2
(Figure 6) follows the attention deviation as the recompute ratio grows,
Figure 7 shows how the KV deviation is distributed over the tokens of a layer,
and section 4.3 (Figure 8) measures how similar the KV deviation is between
neighbouring layers with Spearman's rank correlation.  Written from those
definitions with numpy, fp64.
"""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np


def attention_matrix(q: np.ndarray, k_all: np.ndarray, last_key: Sequence[int]) -> np.ndarray:
    """Forward attention matrix of the rows q [m][n_q][hd] over keys k_all
    [T][n_kv][hd]: P[i][h][t] = softmax over t <= last_key[i] of
    q[i,h] . k[t, h // (n_q/n_kv)] / sqrt(hd); 0 for t > last_key[i]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k_all, np.float64)
    m, n_q, hd = q.shape
    T, n_kv, _ = k.shape
    g = n_q // n_kv
    out = np.zeros((m, n_q, T))
    for i in range(m):
        L = int(last_key[i]) + 1
        for h in range(n_q):
            s = k[:L, h // g, :] @ q[i, h] / math.sqrt(hd)
            e = np.exp(s - s.max())
            out[i, h, :L] = e / e.sum()
    return out


def attention_deviation(a: np.ndarray, a_full: np.ndarray) -> float:
    """L-2 (Frobenius) norm of the difference of two attention matrices."""
    d = np.asarray(a, np.float64) - np.asarray(a_full, np.float64)
    return float(np.sqrt(np.sum(d * d)))


def ranks(x: np.ndarray) -> np.ndarray:
    """1-based ranks of x in ascending order; tied values share the mean of
    the ranks they span."""
    x = np.asarray(x, np.float64)
    order = np.argsort(x, kind="stable")
    r = np.empty(len(x))
    i = 0
    while i < len(x):
        j = i
        while j + 1 < len(x) and x[order[j + 1]] == x[order[i]]:
            j += 1
        r[order[i:j + 1]] = (i + j) / 2.0 + 1.0
        i = j + 1
    return r


def spearman(x: np.ndarray, y: np.ndarray) -> float:
    """Spearman's rank correlation: Pearson's correlation of the ranks."""
    rx, ry = ranks(x), ranks(y)
    rx -= rx.mean()
    ry -= ry.mean()
    den = math.sqrt(float(np.sum(rx * rx)) * float(np.sum(ry * ry)))
    return float(np.sum(rx * ry) / den) if den > 0 else float("nan")


def top_share(dev: np.ndarray, frac: float) -> float:
    """Share of the summed deviation held by the ceil(frac * n) tokens of
    highest deviation (how concentrated the KV deviation is, Figure 7)."""
    d = np.sort(np.asarray(dev, np.float64))[::-1]
    n = int(math.ceil(frac * len(d) - 1e-9))
    tot = float(np.sum(d))
    return float(np.sum(d[:n]) / tot) if tot > 0 else float("nan")
