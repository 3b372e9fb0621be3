"""The packed gate/up operand (cb_pack_gateup): its layout against a numpy
re-layout of the weights (bit for bit), and the layer calls with the packed
copy against the same calls on the row-major weights (every output bit for
bit: only the addresses the kernel loads from change, not the order of any
sum).  Ragged cases: an FFN width that is not a multiple of the 112-feature
tile, and a model width that is not a multiple of the 32-element K step."""
import numpy as np
import pytest

from rag_kv_cache_layer_amd import fusor as F
from rag_kv_cache_layer_amd import synth
from tests.gpu_util import dev, host, need_gpu, single_layer_case, torch

pytestmark = pytest.mark.gpu

MED64 = synth.scaled(synth.PRESETS["llama8b_layer"], 1024, 16, 4, 64, 2776, [100, 77, 150], 13)
ODD_D = synth.scaled(synth.PRESETS["llama8b_layer"], 520, 8, 2, 64, 392, [40, 33, 50], 7)


TILE = 112   # features per gate/up tile (224 rows: the gate rows, then the same up rows)


def _layout(gate, up, K):
    """numpy: tiles of 112 features x 32-element steps, 112 gate rows then the
    same 112 up rows per (tile, step) block, zero past the ends."""
    F_, = gate.shape[:1]
    tiles, nk = -(-F_ // TILE), -(-K // 32)
    out = np.zeros((tiles, nk, 2 * TILE, 32), np.uint16)
    g = np.zeros((tiles * TILE, nk * 32), np.uint16)
    u = np.zeros_like(g)
    g[:F_, :K] = gate
    u[:F_, :K] = up
    for t in range(tiles):
        for s in range(nk):
            out[t, s, :TILE] = g[t * TILE:(t + 1) * TILE, s * 32:(s + 1) * 32]
            out[t, s, TILE:] = u[t * TILE:(t + 1) * TILE, s * 32:(s + 1) * 32]
    return out.reshape(-1)


@pytest.mark.parametrize("p", [MED64, ODD_D], ids=["ffn2776", "d520"])
def test_pack_layout(p):
    need_gpu()
    w = synth.layer_weights(p, 0, 0)
    cfg = F.config_of(p)
    layer = F.DeviceLayer(cfg, w).pack_gateup()
    torch.cuda.synchronize()
    got = layer.t["w_gateup_packed"].cpu().numpy().view(np.uint16)
    bits = lambda t: layer.t[t].cpu().view(torch.int16).numpy().view(np.uint16)
    want = _layout(bits("w_gate"), bits("w_up"), p.d_model)
    assert got.size == want.size and np.array_equal(got, want)


def _run(cfg, layer, p, case, s_in, k, ws, rope):
    T, n_ctx, L0 = p.T, p.n_ctx, case["L0"]
    kc, vc = dev(case["k"], torch.bfloat16), dev(case["v"], torch.bfloat16)
    m_in = len(s_in)
    m_out = F.expected_m_out(T, n_ctx, m_in, k)
    hout = torch.zeros((m_out, p.d_model), dtype=torch.bfloat16, device="cuda")
    dv = torch.zeros(m_in, dtype=torch.float32, device="cuda")
    so = torch.zeros(m_out, dtype=torch.int32, device="cuda")
    s_t = dev(np.asarray(s_in, np.int32), torch.int32)
    F.blend_layer(cfg, layer, rope, kc, vc, T, n_ctx, L0, s_t, m_in, dev(case["hidden"], torch.bfloat16), s_t, k,
                  hout, dv, so, ws)
    torch.cuda.synchronize()
    return [host(kc), host(vc), host(hout), np.nan_to_num(host(dv), nan=-1.0), so.cpu().numpy()]


@pytest.mark.parametrize("p", [MED64, ODD_D], ids=["ffn2776", "d520"])
def test_packed_layer_bit_identical(p):
    need_gpu()
    case = single_layer_case(p, 1, prepass_inputs=False)
    cfg = F.config_of(p)
    plain = F.DeviceLayer(cfg, case["w"])
    packed = F.DeviceLayer(cfg, case["w"]).pack_gateup()
    rope = F.DeviceRope(cfg, p.T)
    ws = F.workspace(cfg, p.T, p.T)
    s_all = np.arange(case["L0"], p.T)
    k = 17
    a = _run(cfg, plain, p, case, s_all, k, ws, rope)
    b = _run(cfg, packed, p, case, s_all, k, ws, rope)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # full prefill too
    outs = []
    for L in (plain, packed):
        kk = torch.zeros((p.T, p.kv_dim), dtype=torch.bfloat16, device="cuda")
        vv = torch.zeros_like(kk)
        y = torch.zeros((p.T, p.d_model), dtype=torch.bfloat16, device="cuda")
        F.full_prefill_layer(cfg, L, rope, dev(case["hidden"], torch.bfloat16), p.T, 0, kk, vv, y, ws)
        torch.cuda.synchronize()
        outs.append([host(kk), host(vv), host(y)])
    for x, y in zip(*outs):
        assert np.array_equal(x, y)


def test_packed_full_size_8b_bit_identical():
    """The 8B layer at full size (the launch bench.py times, with the packed
    operand): the blend call equals the row-major call bit for bit."""
    need_gpu()
    p = synth.PRESETS["llama8b_layer"]
    cfg = F.config_of(p)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    shapes = {"w_q": (p.q_dim, p.d_model), "w_k": (p.kv_dim, p.d_model), "w_v": (p.kv_dim, p.d_model),
              "w_o": (p.d_model, p.q_dim), "w_gate": (p.ffn_dim, p.d_model), "w_up": (p.ffn_dim, p.d_model),
              "w_down": (p.d_model, p.ffn_dim)}
    w = {n: (torch.randn(s, generator=g, device="cuda") * 0.02).to(torch.bfloat16) for n, s in shapes.items()}
    w["attn_norm"] = torch.ones(p.d_model, device="cuda")
    w["mlp_norm"] = torch.ones(p.d_model, device="cuda")
    plain = F.DeviceLayer(cfg, w)
    packed = F.DeviceLayer(cfg, w).pack_gateup()
    T, n_ctx = p.T, p.n_ctx
    offs = synth.chunk_offsets(p, range(p.n_chunks))
    L0 = int(offs[1])
    case = {"k": torch.randn((T, p.n_kv_heads, p.head_dim), generator=g, device="cuda").to(torch.bfloat16).cpu()
            .float().numpy(),
            "v": torch.randn((T, p.n_kv_heads, p.head_dim), generator=g, device="cuda").to(torch.bfloat16).cpu()
            .float().numpy(),
            "hidden": torch.randn((T, p.d_model), generator=g, device="cuda").to(torch.bfloat16).cpu().float().numpy(),
            "L0": L0}
    rope = F.DeviceRope(cfg, T)
    ws = F.workspace(cfg, T, T)
    k = F.num_selected(p.r_e4, n_ctx, n_ctx - L0)
    rng = np.random.default_rng(2)
    S = np.concatenate([np.sort(rng.choice(np.arange(L0, n_ctx), k, replace=False)), np.arange(n_ctx, T)])
    a = _run(cfg, plain, p, case, S, k, ws, rope)
    b = _run(cfg, packed, p, case, S, k, ws, rope)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
