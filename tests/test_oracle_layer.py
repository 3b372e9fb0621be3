"""Pins of the oracle's decoder layer: an independent PyTorch-CPU fp64 Llama
layer (SDPA attention, complex RoPE), dense masked attention, and the
prefix-caching invariant (CPU only)."""
import numpy as np
import pytest

from oracle import layer
from rag_kv_cache_layer_amd import synth
from tests import torch_ref

# small shapes: MHA (the tiny fp32 workload) and a GQA shape of the 8B family
TINY = synth.PRESETS["tiny_f32"]
GQA = synth.scaled(synth.PRESETS["llama8b_layer"], 128, 8, 2, 16, 344, [24, 20, 28], 8).with_(dtype="f32")


def _weights64(p, seed):
    return {k: v.astype(np.float64) for k, v in synth.layer_weights(p, seed, 0).items()}


@pytest.mark.parametrize("p", [TINY, GQA], ids=["mha", "gqa"])
@pytest.mark.parametrize("pos0", [0, 37])
def test_full_prefill_matches_torch_fp64(p, pos0):
    w = _weights64(p, 5)
    x = synth.context_embeddings(p, 5, synth.chunk_order(p, 5)).astype(np.float64)
    k, v, y = layer.full_prefill(w, x, p, pos0=pos0)
    k_r, v_r, y_r = torch_ref.layer(w, x, p, pos0=pos0)
    # the oracle's RoPE table is fp32-rounded, the reference's angles are fp64
    assert torch_ref.rel_err(k, k_r) < 2e-6
    assert torch_ref.rel_err(v, v_r) < 1e-12
    assert torch_ref.rel_err(y, y_r) < 2e-6


def test_full_prefill_fp32_close_to_fp64():
    p = GQA
    w = synth.layer_weights(p, 6, 0)
    x = synth.context_embeddings(p, 6, synth.chunk_order(p, 6))
    k, v, y = layer.full_prefill(w, x, p)
    _, _, y_r = torch_ref.layer({a: b.astype(np.float64) for a, b in w.items()}, x.astype(np.float64), p)
    assert y.dtype == np.float32
    assert torch_ref.rel_err(y, y_r) < 1e-5


def test_partial_attention_equals_rows_of_dense_masked_attention():
    p = GQA
    T = 80
    q = synth.random_normal(p, 7, (T, p.n_q_heads, p.head_dim), tag_layer=1).astype(np.float64)
    k = synth.random_normal(p, 7, (T, p.n_kv_heads, p.head_dim), tag_layer=2).astype(np.float64)
    v = synth.random_normal(p, 7, (T, p.n_kv_heads, p.head_dim), tag_layer=3).astype(np.float64)
    rows = synth.random_subset(p, 7, 0, T, 23)
    ours = layer.attention_rows(q[rows], k, v, rows)
    dense = torch_ref.attention_masked(q, k, v, np.arange(T))
    assert torch_ref.rel_err(ours, dense[rows]) < 1e-12
    # arbitrary per-row key limits as well
    last = (rows * 7) % T
    ours2 = layer.attention_rows(q[rows], k, v, last)
    ref2 = torch_ref.attention_masked(q[rows], k, v, last)
    assert torch_ref.rel_err(ours2, ref2) < 1e-12


def test_single_key_attention_returns_that_value():
    p = GQA
    q = synth.random_normal(p, 8, (3, p.n_q_heads, p.head_dim))
    k = synth.random_normal(p, 8, (5, p.n_kv_heads, p.head_dim), tag_layer=1)
    v = synth.random_normal(p, 8, (5, p.n_kv_heads, p.head_dim), tag_layer=2)
    o = layer.attention_rows(q, k, v, [0, 0, 0])
    g = p.n_q_heads // p.n_kv_heads
    for h in range(p.n_q_heads):
        assert np.array_equal(o[:, h], np.broadcast_to(v[0, h // g], o[:, h].shape))


@pytest.mark.parametrize("p", [TINY, GQA], ids=["mha", "gqa"])
def test_prefix_invariant_rowwise_bit_exact(p):
    """The prefix chunk's KV and outputs do not depend on what follows it
    (the paper's argument for prefix caching, section 3.2; the ml-canon note:
    the prefix KV is bit-for-bit identical)."""
    w = synth.layer_weights(p, 9, 0)
    x = synth.context_embeddings(p, 9, synth.chunk_order(p, 9))
    L0 = p.chunk_lens[0]
    k0, v0, y0 = layer.full_prefill(w, x[:L0], p, rowwise=True)
    k1, v1, y1 = layer.full_prefill(w, x, p, rowwise=True)
    assert np.array_equal(k0, k1[:L0]) and np.array_equal(v0, v1[:L0]) and np.array_equal(y0, y1[:L0])


def test_store_rounding_is_bf16_rne():
    x = np.array([1.0, 1.00390625, 1.005859375, -3.0e-3, 65504.0], dtype=np.float32)
    r = layer.round_store(x, "bf16")
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1.005859375 = 1 + 1.5 * 2^-8 rounds up
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == np.float32(1.0078125)
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2 ** -8)
