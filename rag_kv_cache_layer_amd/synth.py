"""Seeded synthetic inputs for the CacheBlend fusor layer.

This module draws random numbers and lays out geometry; it holds none of the
method's arithmetic (no RoPE, no projection, no attention, no selection).  Both
the CPU oracle's tests and the GPU path's tests and benchmark read their inputs
from here, so the two sides always start from bit-identical values.

Workload presets follow the RAG setting of the CacheBlend paper (arXiv
2405.16444, section 7.1 "Models and hardware settings" and "Datasets"):
retrieved chunks of 512 tokens in random order, followed by a short query, on
Llama-shaped decoder layers.  Real text, trained weights and the paper's
datasets are not available; every tensor here is a seeded normal draw
(weights N(0, 0.02), hidden states / embeddings N(0, 1), RMSNorm gains 1).

Random streams: numpy ``Generator(PCG64(SeedSequence(seed, spawn_key=key)))``
with ``key = (preset id, tensor tag, layer, chunk id)``; normals are drawn in
fp64, cast to fp32 and, for bf16 presets, rounded to bf16 (round to nearest
even) so that the stored value is exactly representable in both precisions.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

# tensor tags of the spawn key
TAG_WQ, TAG_WK, TAG_WV, TAG_WO, TAG_WGATE, TAG_WUP, TAG_WDOWN = 1, 2, 3, 4, 5, 6, 7
TAG_EMB, TAG_QUERY, TAG_PERM, TAG_MISC = 20, 21, 30, 40

WEIGHT_NAMES = ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down")
_WEIGHT_TAG = dict(zip(WEIGHT_NAMES, (TAG_WQ, TAG_WK, TAG_WV, TAG_WO, TAG_WGATE, TAG_WUP, TAG_WDOWN)))


@dataclasses.dataclass(frozen=True)
class Preset:
    """Shape of one workload.  ``r`` is the recompute ratio in units of 1e-4
    (15% -> 1500) so that token counts derived from it are exact integers."""
    pid: int
    name: str
    dtype: str                  # "f32" or "bf16"
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    rope_theta: float
    n_layers: int
    chunk_lens: tuple
    query_len: int
    r_e4: int                   # recompute ratio x 1e4 at the selecting layer
    r_last_e4: int = 0          # gradual filtering end ratio (0: constant ratio)
    permute_chunks: bool = False
    rms_eps: float = 1e-5

    @property
    def n_chunks(self) -> int:
        return len(self.chunk_lens)

    @property
    def n_ctx(self) -> int:
        return int(sum(self.chunk_lens))

    @property
    def T(self) -> int:
        return self.n_ctx + self.query_len

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    def with_(self, **kw) -> "Preset":
        return dataclasses.replace(self, **kw)


def _p(pid, name, dtype, d, nq, nkv, hd, ffn, theta, layers, chunks, q, r, r_last=0, perm=False):
    return Preset(pid, name, dtype, d, nq, nkv, hd, ffn, float(theta), layers, tuple(chunks), q, r, r_last, perm)


# The five workloads: a tiny fp32 layer, the Llama-3-8B-shaped layer (the
# headline), the 32-layer 8B stack with gradual filtering, the 80-layer
# 70B-shaped stack and the ratio / length sweep on the 8B layer.
PRESETS: Dict[str, Preset] = {
    "tiny_f32": _p(1, "tiny_f32", "f32", 256, 4, 4, 64, 688, 1e4, 1, [64, 64], 16, 1500),
    "llama8b_layer": _p(2, "llama8b_layer", "bf16", 4096, 32, 8, 128, 14336, 5e5, 1, [512] * 6, 32, 1500),
    "llama8b_stack": _p(3, "llama8b_stack", "bf16", 4096, 32, 8, 128, 14336, 5e5, 32, [512] * 8, 64, 3000, 1500),
    "llama70b_stack": _p(4, "llama70b_stack", "bf16", 8192, 64, 8, 128, 28672, 5e5, 80, [500] * 8, 32, 1500),
}


def sweep_preset(n_chunks: int, r_e4: int) -> Preset:
    """Ratio / length sweep on the 8B-shaped layer: n_chunks x 512 + 64 query."""
    return _p(5, f"llama8b_sweep_c{n_chunks}_r{r_e4}", "bf16", 4096, 32, 8, 128, 14336, 5e5, 1,
              [512] * n_chunks, 64, r_e4, 0, True)


def scaled(p: Preset, d_model: int, n_q: int, n_kv: int, head_dim: int, ffn: int,
           chunk_lens: Sequence[int], query_len: int, n_layers: Optional[int] = None) -> Preset:
    """Same workload family at reduced width (used for fast CPU-checkable cases)."""
    return dataclasses.replace(p, d_model=d_model, n_q_heads=n_q, n_kv_heads=n_kv, head_dim=head_dim,
                               ffn_dim=ffn, chunk_lens=tuple(chunk_lens), query_len=query_len,
                               n_layers=p.n_layers if n_layers is None else n_layers,
                               name=p.name + f"_scaled{d_model}")


# --------------------------------------------------------------------------
# bf16 storage helpers (bit manipulation only)
# --------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round an fp32 array to the storage dtype and return it as fp32 values."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy()
    if dtype == "bf16":
        return bf16_to_f32(bf16_bits(x))
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# random streams
# --------------------------------------------------------------------------

def rng(p: Preset, seed: int, tag: int, layer: int = 0, chunk: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(p.pid, tag, layer, chunk))
    return np.random.Generator(np.random.PCG64(ss))


def _normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    out = g.standard_normal(size=shape, dtype=np.float64)
    out *= std
    return out.astype(np.float32)


def layer_weights(p: Preset, seed: int, layer: int, std: float = 0.02) -> Dict[str, np.ndarray]:
    """One decoder layer's weights in nn.Linear layout [out][in], fp32 values
    already rounded to the preset's storage dtype.  Norm gains are 1."""
    shapes = {
        "w_q": (p.q_dim, p.d_model), "w_k": (p.kv_dim, p.d_model), "w_v": (p.kv_dim, p.d_model),
        "w_o": (p.d_model, p.q_dim), "w_gate": (p.ffn_dim, p.d_model), "w_up": (p.ffn_dim, p.d_model),
        "w_down": (p.d_model, p.ffn_dim),
    }
    w = {}
    for name in WEIGHT_NAMES:
        w[name] = round_to(_normal(rng(p, seed, _WEIGHT_TAG[name], layer), shapes[name], std), p.dtype)
    w["attn_norm"] = np.ones(p.d_model, dtype=np.float32)
    w["mlp_norm"] = np.ones(p.d_model, dtype=np.float32)
    return w


def chunk_embedding(p: Preset, seed: int, chunk_id: int) -> np.ndarray:
    """Hidden states / token embeddings of one chunk, N(0, 1), [L_c][d]."""
    L = p.chunk_lens[chunk_id]
    return round_to(_normal(rng(p, seed, TAG_EMB, 0, chunk_id), (L, p.d_model), 1.0), p.dtype)


def query_embedding(p: Preset, seed: int) -> np.ndarray:
    return round_to(_normal(rng(p, seed, TAG_QUERY), (p.query_len, p.d_model), 1.0), p.dtype)


def chunk_order(p: Preset, seed: int) -> List[int]:
    """Context order of the chunk ids (a seeded permutation for the sweep)."""
    ids = list(range(p.n_chunks))
    if p.permute_chunks:
        ids = [int(i) for i in rng(p, seed, TAG_PERM).permutation(p.n_chunks)]
    return ids


def chunk_offsets(p: Preset, order: Sequence[int]) -> np.ndarray:
    """Start row of each chunk in context order, plus n_ctx at the end."""
    lens = [p.chunk_lens[c] for c in order]
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def context_embeddings(p: Preset, seed: int, order: Sequence[int]) -> np.ndarray:
    """Embeddings of the whole input [T][d]: chunks in context order, then the query."""
    parts = [chunk_embedding(p, seed, c) for c in order] + [query_embedding(p, seed)]
    return np.concatenate(parts, axis=0)


def random_subset(p: Preset, seed: int, lo: int, hi: int, k: int, tag_layer: int = 0) -> np.ndarray:
    """k distinct sorted rows drawn uniformly from [lo, hi) (used to build a
    given selection set for kernel-level tests)."""
    g = rng(p, seed, TAG_MISC, tag_layer)
    return np.sort(g.choice(np.arange(lo, hi, dtype=np.int64), size=k, replace=False)).astype(np.int32)


def random_normal(p: Preset, seed: int, shape, std: float = 1.0, tag_layer: int = 0, tag_chunk: int = 0) -> np.ndarray:
    """A generic seeded normal draw, rounded to the storage dtype."""
    return round_to(_normal(rng(p, seed, TAG_MISC, tag_layer, tag_chunk + 1), shape, std), p.dtype)
