"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case monkeypatches one plausible error into ``oracle/`` (a dropped term,
a wrong sign or index, a transposed pairing, an off-by-one) and checks that
the pin test guarding that part now fails."""
import math

import numpy as np
import pytest

from oracle import blend, layer, rope
from tests import test_oracle_blend as tb
from tests import test_oracle_layer as tl
from tests import test_oracle_rope as tr
from tests import test_oracle_select as ts


@pytest.fixture(autouse=True)
def _fresh_tables():
    rope._table.cache_clear()
    yield
    rope._table.cache_clear()


def _fails(fn, *a):
    with pytest.raises(AssertionError):
        fn(*a)


def test_sin_sign_flip_is_caught(monkeypatch):
    orig = rope.rotate
    monkeypatch.setattr(rope, "rotate", lambda x, c, s: orig(x, c, -s))
    _fails(tr.test_rotate_matches_complex_multiplication)


def test_half_split_pairing_is_caught(monkeypatch):
    def half_split(x, cos, sin):
        h = x.shape[-1] // 2
        a, b = x[..., :h], x[..., h:]
        c, s = cos[:, None, :].astype(x.dtype), sin[:, None, :].astype(x.dtype)
        return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)
    monkeypatch.setattr(rope, "rotate", half_split)
    _fails(tr.test_rotate_matches_complex_multiplication)


def test_frequency_exponent_is_caught(monkeypatch):
    monkeypatch.setattr(rope, "inv_freq", lambda th, hd: [math.pow(th, -1.0 * i / hd) for i in range(hd // 2)])
    _fails(tr.test_table_matches_complex_exponential)


def test_shift_by_wrong_offset_is_caught(monkeypatch):
    monkeypatch.setattr(rope, "rope_shift", _shift_plus_one)
    _fails(tr.test_shift_composes_to_absolute_position, np.float64)


def _shift_plus_one(k_cache, offs, theta):
    offs = [int(o) for o in offs]
    out = k_cache.copy()
    for c in range(1, len(offs) - 1):
        lo, hi = offs[c], offs[c + 1]
        cos, sin = rope.rope_table(theta, k_cache.shape[-1], np.full(hi - lo, lo + 1))
        out[lo:hi] = rope.rotate(k_cache[lo:hi], cos, sin)
    return out


def _mutated_attention(head_map=None, extra_keys=0, scale_mul=1.0):
    def attn(q, k_all, v_all, last_key):
        m, n_q, hd = q.shape
        n_kv = k_all.shape[1]
        g = n_q // n_kv
        out = np.empty_like(q)
        for i in range(m):
            L = min(int(last_key[i]) + 1 + extra_keys, k_all.shape[0])
            for h in range(n_q):
                kv = head_map(h, g, n_kv) if head_map else h // g
                s = (k_all[:L, kv] @ q[i, h]) * (scale_mul / math.sqrt(hd))
                e = np.exp(s - s.max())
                out[i, h] = (e / e.sum()) @ v_all[:L, kv]
        return out
    return attn


def test_gqa_head_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(layer, "attention_rows", _mutated_attention(head_map=lambda h, g, n: h % n))
    _fails(tl.test_full_prefill_matches_torch_fp64, tl.GQA, 0)


def test_causal_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(layer, "attention_rows", _mutated_attention(extra_keys=1))
    _fails(tl.test_full_prefill_matches_torch_fp64, tl.TINY, 0)


def test_missing_softmax_scale_is_caught(monkeypatch):
    monkeypatch.setattr(layer, "attention_rows", _mutated_attention(scale_mul=math.sqrt(64)))
    _fails(tl.test_full_prefill_matches_torch_fp64, tl.TINY, 0)


def test_rmsnorm_without_eps_inside_root_is_caught(monkeypatch):
    monkeypatch.setattr(layer, "rmsnorm", lambda x, g, eps: x / (np.sqrt(np.mean(x * x, -1, keepdims=True)) + 0.5) * g)
    _fails(tl.test_full_prefill_matches_torch_fp64, tl.TINY, 0)


def test_swiglu_operands_swapped_is_caught(monkeypatch):
    def out_rows(w, x, o, cfg, rowwise=False, lin=None):
        n = x.shape[0]
        h = x + layer.linear(o.reshape(n, -1), w["w_o"], rowwise)
        hn = layer.rmsnorm(h, w["mlp_norm"], cfg.rms_eps)
        u = layer.linear(hn, w["w_gate"], rowwise) * layer.silu(layer.linear(hn, w["w_up"], rowwise))
        return h + layer.linear(u, w["w_down"], rowwise)
    monkeypatch.setattr(layer, "out_rows", out_rows)
    _fails(tl.test_full_prefill_matches_torch_fp64, tl.GQA, 0)


def test_dropped_attention_residual_is_caught(monkeypatch):
    def out_rows(w, x, o, cfg, rowwise=False, lin=None):
        n = x.shape[0]
        h = layer.linear(o.reshape(n, -1), w["w_o"], rowwise)
        hn = layer.rmsnorm(h, w["mlp_norm"], cfg.rms_eps)
        u = layer.silu(layer.linear(hn, w["w_gate"], rowwise)) * layer.linear(hn, w["w_up"], rowwise)
        return h + layer.linear(u, w["w_down"], rowwise)
    monkeypatch.setattr(layer, "out_rows", out_rows)
    _fails(tl.test_full_prefill_matches_torch_fp64, tl.GQA, 0)


def test_deviation_after_overwrite_is_caught(monkeypatch):
    monkeypatch.setattr(blend, "k_deviation", lambda k_new, k_old: np.zeros(k_new.shape[0], k_new.dtype))
    _fails(tb.test_deviation_taken_before_overwrite)


def test_reversed_tie_break_is_caught(monkeypatch):
    def topk(dev, k):
        n = len(dev)
        k = max(0, min(int(k), n))
        order = sorted(range(n), key=lambda i: (-float(dev[i]), -i))
        return np.array(sorted(order[:k]), dtype=np.int64)
    monkeypatch.setattr(blend, "topk_hkvd", topk)
    _fails(ts.test_topk_brute_force_with_ties)


def test_floor_count_is_caught(monkeypatch):
    monkeypatch.setattr(blend, "num_selected", lambda r, n, c: min(int(r * n / 10000), c))
    _fails(ts.test_num_selected_exact_ceiling)


def test_ascending_selection_is_caught(monkeypatch):
    # picking the LOWEST deviations instead of the highest
    def topk(dev, k):
        n = len(dev)
        k = max(0, min(int(k), n))
        order = sorted(range(n), key=lambda i: (float(dev[i]), i))
        return np.array(sorted(order[:k]), dtype=np.int64)
    monkeypatch.setattr(blend, "topk_hkvd", topk)
    _fails(tb.test_nesting_and_counts_under_gradual_filtering)
