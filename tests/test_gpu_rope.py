"""cb_rope_shift against the oracle's re-rotation (CacheBlend section 4.3,
footnote 3): bit-exact, since both sides compute each output as two rounded
fp32 products and one rounded sum from the same fp32 table, then round to the
cache dtype."""
import numpy as np
import pytest

from oracle import rope
from rag_kv_cache_layer_amd import fusor as F
from rag_kv_cache_layer_amd import synth
from tests.gpu_util import act_dtype, dev, host, need_gpu, store_of, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunks,query,hd,nkv", [([37, 64, 0, 91], 5, 64, 2), ([512] * 6, 32, 128, 8),
                                                 ([1], 0, 64, 1), ([20], 3, 128, 2)])
def test_shift_bit_exact(dtype, chunks, query, hd, nkv):
    _shift_case(dtype, chunks, query, hd, nkv)


@pytest.mark.parametrize("hd,nkv", [(72, 1), (8, 1), (24, 3), (40, 1)])
def test_shift_rows_not_a_multiple_of_16(hd, nkv):
    """fp32 key rows of 72, 8, 72 and 40 elements: every pair is rotated (the
    kernel's unit per thread follows the row length)."""
    _shift_case("f32", [37, 64, 21], 5, hd, nkv)


def _shift_case(dtype, chunks, query, hd, nkv):
    need_gpu()
    p = synth.scaled(synth.PRESETS["llama8b_layer"], 256, nkv * 2, nkv, hd, 512, chunks, query).with_(dtype=dtype)
    cfg = F.config_of(p)
    T, kv = p.T, nkv * hd
    n_layers, stride = 3, T * kv + 64
    offs = synth.chunk_offsets(p, range(len(chunks)))
    base = synth.random_normal(p, 7, (n_layers * stride,), std=1.5)
    buf = dev(base, act_dtype(p))
    r = F.DeviceRope(cfg, T)
    F.rope_shift(cfg, r, buf, stride, n_layers, T, offs)
    torch.cuda.synchronize()
    got = host(buf)
    for l in range(n_layers):
        k = base[l * stride:l * stride + T * kv].reshape(T, nkv, hd)
        want = rope.rope_shift(k, offs, p.rope_theta, store_of(p))
        g = got[l * stride:l * stride + T * kv].reshape(T, nkv, hd)
        assert np.array_equal(g.view(np.uint32), want.view(np.uint32)), l
        # padding between layers is never touched
        assert np.array_equal(got[l * stride + T * kv:(l + 1) * stride], base[l * stride + T * kv:(l + 1) * stride])


def test_shift_closed_form_and_stack_size():
    """32-layer 8B-shaped stack (8 x 512 + 64 tokens): every layer bit-exact vs
    the oracle, chunk 0 and query rows untouched, and the shifted key equals
    the key rotated directly at its absolute position within fp32 rounding."""
    need_gpu()
    p = synth.PRESETS["llama8b_stack"]
    cfg = F.config_of(p)
    T, kv, n_layers = p.T, p.kv_dim, p.n_layers
    offs = synth.chunk_offsets(p, range(p.n_chunks))
    base = synth.random_normal(p, 3, (n_layers, T, p.n_kv_heads, p.head_dim))
    buf = dev(base, torch.bfloat16)
    r = F.DeviceRope(cfg, T)
    F.rope_shift(cfg, r, buf, T * kv, n_layers, T, offs)
    torch.cuda.synchronize()
    got = host(buf)
    for l in range(n_layers):
        want = rope.rope_shift(base[l], offs, p.rope_theta, "bf16")
        assert np.array_equal(got[l].view(np.uint32), want.view(np.uint32)), l
    assert np.array_equal(got[:, :512], base[:, :512])
    assert np.array_equal(got[:, p.n_ctx:], base[:, p.n_ctx:])
    # closed form R(m + delta) = R(delta) R(m): a raw key rotated at local m
    # then shifted equals the raw key rotated at m + delta (fp32, no storage rounding)
    raw = synth.random_normal(p.with_(dtype="f32"), 4, (T, p.n_kv_heads, p.head_dim))
    local = np.concatenate([np.arange(L) for L in p.chunk_lens] + [np.arange(p.query_len)])
    cached = rope.apply_rope(raw, local, p.rope_theta)
    cfg32 = F.config_of(p.with_(dtype="f32"))
    b32 = dev(cached, torch.float32)
    F.rope_shift(cfg32, F.DeviceRope(cfg32, T), b32, T * kv, 1, T, offs)
    torch.cuda.synchronize()
    absolute = rope.apply_rope(raw[:p.n_ctx], np.arange(p.n_ctx), p.rope_theta)
    g = host(b32)[:p.n_ctx]
    assert np.max(np.abs(g - absolute)) <= 1e-5 * np.max(np.abs(absolute)) * 8
