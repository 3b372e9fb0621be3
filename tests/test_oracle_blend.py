"""Pins of the oracle's fusor: r = 1 equals full prefill, the prefix-caching
special case, gather/scatter, nesting and counts, the shift-only deviation,
and the single-layer input construction (CPU only)."""
import numpy as np
import pytest

from oracle import blend, layer, prepass, rope
from rag_kv_cache_layer_amd import synth
from tests import torch_ref

GQA = synth.scaled(synth.PRESETS["llama8b_layer"], 128, 8, 2, 16, 344, [24, 20, 28], 8).with_(dtype="f32")
TINY = synth.PRESETS["tiny_f32"]


def _stack_case(p, seed, n_layers, rowwise=True, store=None):
    ws = [synth.layer_weights(p, seed, l) for l in range(n_layers)]
    order = synth.chunk_order(p, seed)
    offs = synth.chunk_offsets(p, order)
    kv = {c: blend.precompute_chunk(ws, p, synth.chunk_embedding(p, seed, c), rowwise, store) for c in order}
    K, V = blend.assemble_caches(p, kv, order, p.T, n_layers)
    K = blend.shift_caches(p, K, offs)
    x_all = synth.context_embeddings(p, seed, order)
    return ws, offs, K, V, x_all


@pytest.mark.parametrize("p", [TINY, GQA], ids=["mha", "gqa"])
def test_ratio_one_stack_equals_full_prefill(p):
    """Recomputing every token on every layer is full prefill (section 4.2:
    compute is r% of full prefill; r = 100% is the full KV recompute baseline)."""
    n_layers = 3
    ws, offs, K, V, x_all = _stack_case(p, 11, n_layers)
    L0, n_ctx = int(offs[1]), int(offs[-1])
    n_cand = n_ctx - L0
    res = blend.blend_stack(ws, p, K, V, n_ctx, L0, x_all, [n_cand] * n_layers, rowwise=True)
    Kf, Vf, yf = blend.full_prefill_stack(ws, p, x_all, rowwise=True)
    for l in range(n_layers):
        assert np.array_equal(res["K"][l], Kf[l]), l
        assert np.array_equal(res["V"][l], Vf[l]), l
    assert np.array_equal(res["s_last"], np.arange(L0, p.T))
    assert np.array_equal(res["y"], yf[L0:])


def test_ratio_one_blas_mode_close():
    p = GQA
    ws, offs, K, V, x_all = _stack_case(p, 12, 2, rowwise=False)
    L0, n_ctx = int(offs[1]), int(offs[-1])
    res = blend.blend_stack(ws, p, K, V, n_ctx, L0, x_all, [n_ctx - L0] * 2)
    Kf, Vf, yf = blend.full_prefill_stack(ws, p, x_all)
    assert torch_ref.rel_err(res["y"], yf[L0:]) < 1e-5
    assert torch_ref.rel_err(res["K"][1], Kf[1]) < 1e-5


def test_prefix_caching_special_case():
    """One cached chunk and nothing recomputed in it: the query rows' outputs
    equal full prefill (prefix caching is CacheBlend with r = 0 on the prefix)."""
    p = GQA.with_(chunk_lens=(40,), query_len=8)
    ws, offs, K, V, x_all = _stack_case(p, 13, 2)
    res = blend.blend_stack(ws, p, K, V, 40, 40, x_all, [0, 0], rowwise=True)
    Kf, Vf, yf = blend.full_prefill_stack(ws, p, x_all, rowwise=True)
    assert np.array_equal(res["y"], yf[40:])
    assert np.array_equal(res["K"][1], Kf[1]) and np.array_equal(res["V"][1], Vf[1])


def test_full_reuse_degenerate_case_runs():
    p = GQA
    ws, offs, K, V, x_all = _stack_case(p, 14, 2, rowwise=False)
    L0, n_ctx = int(offs[1]), int(offs[-1])
    res = blend.blend_stack(ws, p, K, V, n_ctx, L0, x_all, [0, 0])
    assert np.array_equal(res["s_last"], np.arange(n_ctx, p.T))
    # layer 1 recomputed only the query rows: every context row is the shifted cache
    assert np.array_equal(res["K"][1][:n_ctx], K[1][:n_ctx])


def test_gather_scatter_rows():
    p = GQA
    ws, offs, K, V, x_all = _stack_case(p, 15, 1, rowwise=False)
    L0, n_ctx = int(offs[1]), int(offs[-1])
    s_in = np.concatenate([synth.random_subset(p, 15, L0, n_ctx, 17), np.arange(n_ctx, p.T)])
    x = x_all[s_in]
    r = blend.blend_layer(ws[0], p, K[0], V[0], n_ctx, s_in, x, 9)
    untouched = np.setdiff1d(np.arange(p.T), s_in)
    assert np.array_equal(r["k_cache"][untouched], K[0][untouched])
    assert np.array_equal(r["v_cache"][untouched], V[0][untouched])
    _, k_new, v_new = layer.qkv_rows(ws[0], x, s_in, p)
    assert np.array_equal(r["k_cache"][s_in], k_new) and np.array_equal(r["v_cache"][s_in], v_new)
    assert len(r["s_out"]) == 9 + p.query_len and np.all(np.diff(r["s_out"]) > 0)
    assert np.all(np.isnan(r["dev"][-p.query_len:])) and np.all(np.isfinite(r["dev"][:-p.query_len]))


def test_nesting_and_counts_under_gradual_filtering():
    p = GQA
    n_layers = 5
    ws, offs, K, V, x_all = _stack_case(p, 16, n_layers, rowwise=False)
    L0, n_ctx = int(offs[1]), int(offs[-1])
    ks = blend.filter_schedule(n_layers, 5000, 2000, n_ctx, n_ctx - L0)
    # n_ctx = 72: r = 0.5, 0.4, 0.3, 0.2 on layers 1..4 -> ceil(36, 28.8, 21.6, 14.4)
    assert ks == [48, 36, 29, 22, 15]
    res = blend.blend_stack(ws, p, K, V, n_ctx, L0, x_all, ks)
    for l in range(1, n_layers):
        prev, cur = set(res["S"][l - 1].tolist()), set(res["S"][l].tolist())
        assert cur <= prev
        assert len(cur) == ks[l - 1] + p.query_len
    # the kept rows of a selecting layer have the largest deviations there
    dev1, s1, s2 = res["dev"][1], res["S"][1], set(res["S"][2].tolist())
    kept = np.array([s in s2 for s in s1[:len(s1) - p.query_len]])
    d = dev1[:len(s1) - p.query_len]
    assert d[kept].min() >= d[~kept].max()


def test_shift_only_deviation_is_rounding():
    """Literal reading: the same hidden states feed the isolated precompute and
    the blended call, so the K deviation is the shift's rounding alone."""
    p = GQA
    w = synth.layer_weights(p, 17, 0)
    order = synth.chunk_order(p, 17)
    offs = synth.chunk_offsets(p, order)
    x_all = synth.context_embeddings(p, 17, order)
    T, n_ctx, L0 = p.T, int(offs[-1]), int(offs[1])
    K = np.zeros((T, p.n_kv_heads, p.head_dim), np.float32)
    V = np.zeros_like(K)
    for c in range(len(order)):
        lo, hi = int(offs[c]), int(offs[c + 1])
        _, k, v = layer.qkv_rows(w, x_all[lo:hi], np.arange(hi - lo), p)
        K[lo:hi], V[lo:hi] = k, v
    K = rope.rope_shift(K, offs, p.rope_theta)
    s_in = np.arange(L0, T)
    r = blend.blend_layer(w, p, K, V, n_ctx, s_in, x_all[s_in], 5)
    d = r["dev"][: n_ctx - L0]
    kn = np.sum(r["k_cache"][L0:n_ctx].astype(np.float64).reshape(n_ctx - L0, -1) ** 2, axis=1)
    assert np.max(np.sqrt(d / kn)) < 1e-6
    # V needs no position correction: it is reproduced exactly up to matmul order
    assert torch_ref.rel_err(r["v_cache"][L0:n_ctx], V[L0:n_ctx]) < 1e-6


def test_deviation_taken_before_overwrite():
    p = GQA
    w = synth.layer_weights(p, 18, 0)
    order = synth.chunk_order(p, 18)
    e = [synth.chunk_embedding(p, 18, c) for c in order]
    inp = prepass.single_layer_inputs(w, p, e, synth.query_embedding(p, 18))
    offs = inp["offsets"]
    L0, n_ctx = int(offs[1]), int(offs[-1])
    K = rope.rope_shift(inp["k_pre"], offs, p.rope_theta)
    s_in = np.arange(L0, p.T)
    r = blend.blend_layer(w, p, K, inp["v_pre"], n_ctx, s_in, inp["hidden"][s_in], 10)
    kf, _, _ = layer.full_prefill(w, inp["hidden"], p)
    want = np.sum((kf[L0:n_ctx] - K[L0:n_ctx]).reshape(n_ctx - L0, -1).astype(np.float64) ** 2, axis=1)
    got = r["dev"][: n_ctx - L0]
    assert np.all(got > 0)
    assert np.max(np.abs(got - want) / want) < 1e-4


def test_single_layer_inputs_are_layer_one_of_tied_stack():
    p = GQA
    seed = 19
    w = synth.layer_weights(p, seed, 0)
    order = synth.chunk_order(p, seed)
    offs = synth.chunk_offsets(p, order)
    e = [synth.chunk_embedding(p, seed, c) for c in order]
    inp = prepass.single_layer_inputs(w, p, e, synth.query_embedding(p, seed), rowwise=True)
    L0, n_ctx = int(offs[1]), int(offs[-1])
    k = blend.num_selected(1500, n_ctx, n_ctx - L0)
    s_in = np.arange(L0, p.T)
    K = rope.rope_shift(inp["k_pre"], offs, p.rope_theta)
    one = blend.blend_layer(w, p, K, inp["v_pre"], n_ctx, s_in, inp["hidden"][s_in], k, rowwise=True)
    # the same through the stack driver with layers [W, W]
    kv = {c: blend.precompute_chunk([w, w], p, synth.chunk_embedding(p, seed, c), True) for c in order}
    KK, VV = blend.assemble_caches(p, kv, order, p.T, 2)
    KK = blend.shift_caches(p, KK, offs)
    st = blend.blend_stack([w, w], p, KK, VV, n_ctx, L0, synth.context_embeddings(p, seed, order),
                           [n_ctx - L0, k], rowwise=True)
    assert np.array_equal(st["s_last"], one["s_out"])
    assert np.array_equal(st["y"], one["y"])
    assert np.array_equal(st["K"][1], one["k_cache"])
