"""Pins of the oracle's 8-bit float format (OCP E4M3) and row scaling (CPU).

* The value table: 0, the smallest subnormal 2^-9, the smallest normal 2^-6,
  1 = 0x38, 448 = 0x7E the largest, 0x7F and 0xFF not finite; the 254 finite
  codes decode to distinct values apart from +-0.
* Encoding: every finite code's value maps back to that code (exact values
  round trip); values between two neighbours go to the nearer one; a value
  halfway between two neighbours goes to the one with the even code; the sign
  is kept.  Checked against a brute-force nearest search on random inputs.
* Row exponents: amax <= 448 * 2^e and amax > 448 * 2^(e-1) (smallest e), for
  random rows and for the edge cases amax = 448 * 2^k (exact fit) and just
  above; an all-zero row gets 0.
* The GEMM of quantized operands equals the brute-force sum of products of
  the decoded values.
* Stored KV: a cache already on the scaled E4M3 grid survives quantize ->
  expand bit for bit (expansion is exact), each (token, head) row gets its
  own exponent, hand-built codes decode to their values, and any cache comes
  back within half a quantum of its row's binade; the expanded values are
  bf16 numbers."""
import numpy as np
import pytest

from oracle import blend, fp8, layer
from rag_kv_cache_layer_amd import synth


def test_value_table():
    v = fp8.VALUES
    assert v[0x00] == 0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.nanmax(v) == 448.0 and np.nanmin(v) == -448.0
    finite = v[~np.isnan(v)]
    assert len(finite) == 254 and len(np.unique(finite)) == 253   # +0 and -0


def test_encode_round_trip_and_nearest():
    codes = np.array([c for c in range(256) if not np.isnan(fp8.VALUES[c])], np.uint8)
    back = fp8.encode(fp8.VALUES[codes])
    assert np.array_equal(fp8.VALUES[back], fp8.VALUES[codes])
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-1, 1, 4000) * 2.0 ** -5,
                        rng.normal(0, 3, 4000)])
    y = np.clip(y, -448, 448)
    got = fp8.VALUES[fp8.encode(y)]
    grid = np.unique(fp8.VALUES[~np.isnan(fp8.VALUES)])
    d = np.abs(grid[None, :] - y[:, None])
    assert np.all(np.abs(got - y) == d.min(axis=1))


def test_ties_go_to_even_code():
    grid = np.unique(fp8.VALUES[~np.isnan(fp8.VALUES)])
    pos = grid[grid >= 0]
    mids = (pos[:-1] + pos[1:]) / 2
    c = fp8.encode(mids)
    assert np.all((c & 1) == 0)
    assert np.all(fp8.encode(-mids) == (c | 0x80))


def test_row_exponents_smallest_fit():
    rng = np.random.default_rng(1)
    x = (rng.normal(size=(50, 33)) * np.exp(rng.uniform(-20, 20, (50, 1)))).astype(np.float32)
    e = fp8.row_exponents(x)
    amax = np.abs(x).max(1).astype(np.float64)
    assert np.all(amax <= 448 * 2.0 ** e) and np.all(amax > 448 * 2.0 ** (e - 1))
    edge = np.array([[448.0], [896.0], [np.nextafter(np.float32(448.0), np.float32(1e9))], [0.0], [1.0]], np.float32)
    assert list(fp8.row_exponents(edge)) == [0, 1, 1, 0, -8]


def test_quantized_gemm_is_the_sum_of_decoded_products():
    rng = np.random.default_rng(2)
    a = rng.normal(size=(3, 40)).astype(np.float32)
    b = rng.normal(size=(5, 40)).astype(np.float32) * 0.02
    qa, ea = fp8.quantize_rows(a)
    qb, eb = fp8.quantize_rows(b)
    c = fp8.gemm(qa, ea, qb, eb)
    for i in range(3):
        for j in range(5):
            s = sum(fp8.VALUES[qa[i, k]] * 2.0 ** ea[i] * fp8.VALUES[qb[j, k]] * 2.0 ** eb[j] for k in range(40))
            assert c[i, j] == pytest.approx(s, rel=1e-12, abs=1e-15)
    # the quantization error is within half a quantum of each value's binade
    assert np.max(np.abs(fp8.dequantize_rows(qa, ea) - a) / np.abs(a).max(1, keepdims=True)) <= 2.0 ** -4


def test_kv_expand_exact_and_per_head_scale():
    rng = np.random.default_rng(3)
    T, H, D = 9, 3, 16
    # values already on the grid, each (token, head) row with its own scale
    codes = rng.integers(0, 0x7E, size=(T, H, D)).astype(np.uint8) | (rng.integers(0, 2, (T, H, D)) << 7).astype(np.uint8)
    codes[..., 0] = 0x7E                                   # every row reaches 448: exponent = the row's scale
    e = rng.integers(-20, 20, size=(T, H)).astype(np.int32)
    x = (fp8.VALUES[codes] * 2.0 ** e[..., None]).astype(np.float32)
    c2, e2 = fp8.quantize_kv(x)
    assert np.array_equal(e2, e)
    assert np.array_equal(fp8.VALUES[c2], fp8.VALUES[codes])
    back = fp8.expand_kv(c2, e2)
    assert back.dtype == np.float32 and np.array_equal(back, x)
    # hand-built codes: 0x38 = 1, 0x01 = 2^-9, 0xC0 = -2 at the row scales below
    hc = np.zeros((1, 2, 16), np.uint8)
    hc[0, 0, :3] = [0x38, 0x01, 0xC0]
    hc[0, 1, :3] = [0x38, 0x01, 0xC0]
    he = np.array([[0, 5]], np.int32)
    v = fp8.expand_kv(hc, he)
    assert list(v[0, 0, :3]) == [1.0, 2.0 ** -9, -2.0] and list(v[0, 1, :3]) == [32.0, 2.0 ** -4, -64.0]
    # any cache: within half a quantum of the row's binade; bf16-representable
    y = (rng.normal(size=(T, H, D)) * np.exp(rng.uniform(-8, 8, (T, H, 1)))).astype(np.float32)
    cy, ey = fp8.quantize_kv(y)
    z = fp8.expand_kv(cy, ey)
    assert np.all(np.abs(z - y) <= 2.0 ** -4 * np.abs(y).max(2, keepdims=True))
    u = z.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)


def _codes(rng, rows, cols):
    c = rng.integers(0x10, 0x70, size=(rows, cols)).astype(np.uint8)
    c |= (rng.integers(0, 2, size=(rows, cols)) << 7).astype(np.uint8)
    return c, rng.integers(-6, 3, size=rows).astype(np.int32)


def test_projector_exact_on_the_grid_and_rounds_activations():
    rng = np.random.default_rng(4)
    wc, we = _codes(rng, 16, 32)
    xc, xe = _codes(rng, 5, 32)
    xc[:, 0] = 0x7E                                       # each row reaches 448 * 2^e: its exponent is e
    x = fp8.dequantize_rows(xc, xe).astype(np.float32)    # E4M3 values are bf16 numbers
    lin = fp8.projector({"w_o": (wc, we)}, "bf16")
    want = (x.astype(np.float64) @ fp8.dequantize_rows(wc, we).T).astype(np.float32)
    assert np.array_equal(lin(x, "w_o"), want)
    # activations are rounded to bf16 first: 1.1875 - 2^-12 rounds to 1.125 in
    # E4M3 directly, but bf16 rounds it to 1.1875, the E4M3 midpoint of 1.125
    # and 1.25, whose tie goes to the even code (1.25)
    y = np.zeros((1, 32), np.float32)
    y[0, 0] = 448.0                                       # row exponent 0
    y[0, 1] = np.float32(1.1875 - 2.0 ** -12)
    one_hot = np.zeros((32, 32), np.uint8)
    one_hot[np.arange(32), np.arange(32)] = 0x38          # the identity (1.0) as codes
    ident = fp8.projector({"w_o": (one_hot, np.zeros(32, np.int32))}, "bf16")
    got = ident(y, "w_o")
    assert got[0, 0] == 448.0 and got[0, 1] == 1.25
    raw = fp8.projector({"w_o": (one_hot, np.zeros(32, np.int32))}, None)
    assert raw(y, "w_o")[0, 1] == 1.125


def test_fp8_layer_close_to_fp32_and_ratio_one_is_its_full_prefill():
    p = synth.PRESETS["tiny_f32"]
    w = synth.layer_weights(p, 0, 0)
    lin = fp8.projector(fp8.quantize_layer(w), "bf16")
    x = synth.random_normal(p, 0, (p.T, p.d_model), tag_layer=13)
    k32, v32, y32 = layer.full_prefill(w, x, p)
    k8, v8, y8 = layer.full_prefill(w, x, p, lin=lin)
    rel = lambda a, b: float(np.max(np.abs(a - b)) / np.max(np.abs(b)))
    for a, b in ((k8, k32), (v8, v32), (y8, y32)):
        assert 1e-3 < rel(a, b) < 0.15
    # r = 1: every candidate recomputed on the 8-bit layer's own full-prefill cache
    L0 = 64
    s_in = np.arange(L0, p.T)
    out = blend.blend_layer(w, p, k8, v8, p.n_ctx, s_in, x[s_in], p.n_ctx, lin=lin)
    assert rel(out["k_cache"], k8) < 1e-5 and rel(out["v_cache"], v8) < 1e-5 and rel(out["y"], y8[L0:]) < 1e-5
