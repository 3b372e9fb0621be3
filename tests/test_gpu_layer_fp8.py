"""cb_blend_layer_fp8 (8-bit E4M3 projections, the paper's 8-bit serving of
section 7) against the oracle's layer with the 8-bit projector
(oracle/fp8.py: each projection's input rows rounded to bf16 as stored, then
quantized per row, times the decoded weights, exact in fp64).

The weights' codes come from the oracle's quantizer (medium cases) or are
drawn directly as codes (the full-size 8B layer: synthetic 8-bit weights,
codes in 0x18 .. 0x57 with random signs and per-row exponents); the GPU only
reads them.  Tolerances as the bf16 layer (2e-2 max-rel per tensor): both
sides quantize the same stored bf16 activations, so codes differ only where
the two sides' fp32 rounding moves a value across a rounding boundary.
Selection is compared exactly (the oracle's top-k of the GPU's deviations)
and the outputs on that selection."""
import numpy as np
import pytest

from oracle import blend, fp8, layer
from oracle.storage import round_store
from rag_kv_cache_layer_amd import fusor as F
from rag_kv_cache_layer_amd import synth
from tests.gpu_util import dev, host, need_gpu, rel_err, single_layer_case, torch
from tests.test_gpu_layer import _check_blend

pytestmark = pytest.mark.gpu
TOL = 2e-2

# bf16, GQA group 8, head_dim 128 (the 70B head layout)
MED128 = synth.scaled(synth.PRESETS["llama70b_stack"], 1024, 8, 1, 128, 2048, [130, 61, 140], 9, n_layers=1)
# bf16, keys past 512 (attention key split)
LONG = synth.scaled(synth.PRESETS["llama8b_layer"], 512, 8, 2, 64, 1024, [300, 400, 500], 20)


def _device_weights(cfg, w, w8):
    cat = lambda names: (np.concatenate([w8[n][0] for n in names]), np.concatenate([w8[n][1] for n in names]))
    return F.DeviceLayerFp8(cfg, {"w_qkv": cat(("w_q", "w_k", "w_v")), "w_o": w8["w_o"],
                                  "w_gu": cat(("w_gate", "w_up")), "w_down": w8["w_down"],
                                  "attn_norm": w["attn_norm"], "mlp_norm": w["mlp_norm"]})


def _blend(cfg, p, L, rope, ws, k_cache, v_cache, s_in, hidden, L0, k_out):
    kc, vc = dev(k_cache, torch.bfloat16), dev(v_cache, torch.bfloat16)
    m_in = len(s_in)
    m_out = F.expected_m_out(p.T, p.n_ctx, m_in, k_out)
    hout = torch.zeros((max(m_out, 1), p.d_model), dtype=torch.bfloat16, device="cuda")
    dv = torch.zeros(max(m_in, 1), dtype=torch.float32, device="cuda")
    so = torch.full((max(m_out, 1),), -1, dtype=torch.int32, device="cuda")
    s_t = dev(np.asarray(s_in, np.int32), torch.int32)
    m = F.blend_layer_fp8(cfg, L, rope, kc, vc, p.T, p.n_ctx, L0, s_t, m_in, hidden, s_t, k_out, hout, dv, so, ws)
    torch.cuda.synchronize()
    assert m == m_out
    return dict(k=host(kc), v=host(vc), y=host(hout)[:m], dev=host(dv)[:m_in], s_out=so.cpu().numpy()[:m])


@pytest.mark.parametrize("p", [MED128, LONG], ids=["bf16_hd128", "bf16_long"])
def test_select_then_blend_fp8(p):
    need_gpu()
    case = single_layer_case(p, 0)
    cfg = F.config_of(p)
    w8 = fp8.quantize_layer(case["w"])
    lin = fp8.projector(w8, "bf16")
    L = _device_weights(cfg, case["w"], w8)
    rope = F.DeviceRope(cfg, p.T)
    ws = F.workspace_fp8(cfg, p.T, p.T)
    T, n_ctx, L0 = p.T, p.n_ctx, case["L0"]
    hidden = dev(case["hidden"], torch.bfloat16)
    k = blend.num_selected(p.r_e4, n_ctx, n_ctx - L0)
    s_in = np.arange(L0, T)
    got = _blend(cfg, p, L, rope, ws, case["k"], case["v"], s_in, hidden, L0, k)
    keep = blend.topk_hkvd(got["dev"][:n_ctx - L0], k)
    assert np.array_equal(got["s_out"], np.concatenate([s_in[keep], np.arange(n_ctx, T)]))
    want = blend.blend_layer(case["w"], p, case["k"], case["v"], n_ctx, s_in, case["hidden"][s_in], k,
                             store="bf16", keep=keep, lin=lin)
    _check_blend(p, case, got, want, s_in)
    # the 8-bit layer differs from the bf16 one by the quantization, visibly
    ref = blend.blend_layer(case["w"], p, case["k"], case["v"], n_ctx, s_in, case["hidden"][s_in], k,
                            store="bf16", keep=keep)
    e8 = rel_err(got["y"], ref["y"])
    print(f"\n{p.name}: 8-bit vs bf16 layer output max-rel difference {e8:.3g}")
    assert 1e-3 < e8 < 0.2
    # blend call on the kept set
    s2 = want["s_out"]
    got2 = _blend(cfg, p, L, rope, ws, case["k"], case["v"], s2, hidden, L0, k)
    want2 = blend.blend_layer(case["w"], p, case["k"], case["v"], n_ctx, s2, case["hidden"][s2], k, store="bf16",
                              lin=lin)
    assert np.array_equal(got2["s_out"], s2)
    _check_blend(p, case, got2, want2, s2)


def _random_codes(rng, rows, cols):
    """Synthetic 8-bit weights: codes 0x18 .. 0x57 (values 2^-4 .. 2^3.9) with
    random signs, one exponent per row in -12 .. -10."""
    c = rng.integers(0x18, 0x58, size=(rows, cols), dtype=np.uint8)
    c |= (rng.integers(0, 2, size=(rows, cols), dtype=np.uint8) << 7)
    return c, rng.integers(-12, -9, size=rows).astype(np.int32)


def test_llama8b_layer_fp8_full_size_sampled():
    """The 8B layer at its full size (6 x 512 + 32 tokens, r = 0.15), blend call
    on a kept set as bench.py times it: K/V on every row, the layer output on
    sampled rows computed by the oracle one by one."""
    need_gpu()
    p = synth.PRESETS["llama8b_layer"]
    cfg = F.config_of(p)
    rng = np.random.default_rng(5)
    d, q, kvd, ffn = p.d_model, p.q_dim, p.kv_dim, p.ffn_dim
    w8 = {"w_q": _random_codes(rng, q, d), "w_k": _random_codes(rng, kvd, d), "w_v": _random_codes(rng, kvd, d),
          "w_o": _random_codes(rng, d, q), "w_gate": _random_codes(rng, ffn, d), "w_up": _random_codes(rng, ffn, d),
          "w_down": _random_codes(rng, d, ffn)}
    w = {"attn_norm": np.ones(d, np.float32), "mlp_norm": np.ones(d, np.float32)}
    L = _device_weights(cfg, w, w8)
    lin = fp8.projector(w8, "bf16")
    T, n_ctx = p.T, p.n_ctx
    offs = synth.chunk_offsets(p, range(p.n_chunks))
    L0 = int(offs[1])
    kv = (p.n_kv_heads, p.head_dim)
    kc = synth.random_normal(p, 1, (T,) + kv, std=1.0, tag_layer=11)
    vc = synth.random_normal(p, 1, (T,) + kv, std=1.0, tag_layer=12)
    x = synth.random_normal(p, 1, (T, d), tag_layer=13)
    k = F.num_selected(p.r_e4, n_ctx, n_ctx - L0)
    # a kept set: k candidates spread over the context, then the query rows
    S = np.concatenate([np.sort(rng.choice(np.arange(L0, n_ctx), k, replace=False)), np.arange(n_ctx, T)])
    rope = F.DeviceRope(cfg, T)
    ws = F.workspace_fp8(cfg, T, T)
    got = _blend(cfg, p, L, rope, ws, kc, vc, S, dev(x, torch.bfloat16), L0, k)
    assert np.array_equal(got["s_out"], S)
    # oracle: Q/K/V of every row of S, deviation, scatter; the output of sampled rows
    xq = x[S]
    q_, k_, v_ = layer.qkv_rows(w, xq, S, p, lin=lin)
    k_ = round_store(k_, "bf16")
    v_ = round_store(v_, "bf16")
    kk, vv = kc.copy(), vc.copy()
    kk[S] = k_
    vv[S] = v_
    assert rel_err(got["k"], kk) < TOL and rel_err(got["v"], vv) < TOL
    dv = blend.k_deviation(k_[:k], kc[S[:k]])
    assert rel_err(got["dev"][:k], dv) < TOL and np.all(np.isnan(got["dev"][k:]))
    m = len(S)
    rows = np.unique(np.concatenate([[0, m - 1, k], np.linspace(0, m - 1, 20).astype(int)]))
    o = layer.attention_rows(q_[rows], kk, vv, S[rows])
    y = round_store(layer.out_rows(w, xq[rows], o, p, lin=lin), "bf16")
    e = rel_err(got["y"][rows], y)
    print(f"\nllama8b_layer 8-bit: sampled output max-rel error {e:.3g}")
    assert e < TOL


def test_fp8_degenerate_cases():
    """k = 0 (only the query is recomputed), k >= candidates (every row) and a
    query-only input, on the 8-bit layer."""
    need_gpu()
    p = LONG
    case = single_layer_case(p, 3, prepass_inputs=False)
    cfg = F.config_of(p)
    w8 = fp8.quantize_layer(case["w"])
    lin = fp8.projector(w8, "bf16")
    L = _device_weights(cfg, case["w"], w8)
    rope = F.DeviceRope(cfg, p.T)
    ws = F.workspace_fp8(cfg, p.T, p.T)
    T, n_ctx, L0 = p.T, p.n_ctx, case["L0"]
    hidden = dev(case["hidden"], torch.bfloat16)
    s_all = np.arange(L0, T)
    for k in (0, n_ctx - L0, n_ctx):
        got = _blend(cfg, p, L, rope, ws, case["k"], case["v"], s_all, hidden, L0, k)
        want = blend.blend_layer(case["w"], p, case["k"], case["v"], n_ctx, s_all, case["hidden"][s_all], k,
                                 store="bf16", keep=None if k else np.zeros(0, np.int64), lin=lin)
        assert np.array_equal(got["s_out"], s_all if k else np.arange(n_ctx, T))
        _check_blend(p, case, got, want, s_all)
    q_only = np.arange(n_ctx, T)
    got = _blend(cfg, p, L, rope, ws, case["k"], case["v"], q_only, hidden, L0, 5)
    want = blend.blend_layer(case["w"], p, case["k"], case["v"], n_ctx, q_only, case["hidden"][q_only], 5,
                             store="bf16", lin=lin)
    assert np.array_equal(got["s_out"], q_only)
    _check_blend(p, case, got, want, q_only)
