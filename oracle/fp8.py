"""8-bit floating-point weights and activations for the oracle (test
infrastructure only).

The paper serves its larger models with 8-bit weights (CacheBlend section 7,
models).  The reading taken here: OCP fp8 E4M3 (1 sign, 4 exponent bits with
bias 7, 3 mantissa bits; largest finite value 448, no infinities) with one
power-of-two scale per matrix row, so that scaling is exact and only the
rounding to E4M3 loses information:

    e    = the smallest integer with amax(row) <= 448 * 2^e
    code = round-to-nearest-even of x * 2^-e onto the E4M3 grid
    x   ~= value(code) * 2^e

A product C = A B^T of two such matrices is then exactly
sum_k value(a_code) value(b_code) * 2^(e_a + e_b); every product of two
E4M3 values is exact in fp32, so only the accumulation order rounds.

Stored KV in this format (the loader of CacheBlend section 5 moves the
chunk KV; 8 bits halve those bytes) is scaled per (token, KV head): the rows
of the quantizer are the head_dim values of one head of one token.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def row_exponents(x: np.ndarray) -> np.ndarray:
    """Per row: the smallest integer e with max|x_row| <= 448 * 2^e (0 for an
    all-zero row).  With amax = m * 2^E, m in [1, 2): e = E - 8 + (m > 1.75)."""
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=1).astype(np.float64)
    out = np.zeros(len(amax), np.int32)
    for i, a in enumerate(amax):
        if a > 0:
            m, E = math.frexp(a)       # a = m * 2^E with m in [0.5, 1)
            m, E = 2 * m, E - 1        # m in [1, 2)
            out[i] = E - 8 + (1 if m > 1.75 else 0)
    return out


def _grid():
    """All finite E4M3 values of the codes 0..255 (NaN codes excluded)."""
    vals = np.full(256, np.nan)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        vals[c] = s * (m / 8.0) * 2.0 ** -6 if e == 0 else s * (1 + m / 8.0) * 2.0 ** (e - 7)
    return vals


VALUES = _grid()


def encode(y: np.ndarray) -> np.ndarray:
    """Round fp32 values already within [-448, 448] to the nearest E4M3 code,
    ties to the even mantissa (the code with an even last bit)."""
    y = np.asarray(y, np.float64)
    a = np.abs(y)
    # the quantum of the binade of |y|: 2^(E-3) for normal values, 2^-9 below 2^-6
    E = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    q = 2.0 ** (E - 3)
    n = a / q
    r = np.floor(n)
    frac = n - r
    r = np.where((frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2) == 1)), r + 1, r)
    mag = r * q
    # encode the magnitude: subnormals (e = 0) and normals
    codes = np.zeros(y.shape, np.uint8)
    sub = mag < 2.0 ** -6
    codes = np.where(sub, np.round(mag / 2.0 ** -9).astype(np.int64), 0)
    Em = np.floor(np.log2(np.where(sub, 1.0, mag)))
    mant = np.where(sub, 0, np.round((mag / 2.0 ** Em - 1.0) * 8).astype(np.int64))
    norm = ((Em.astype(np.int64) + 7) << 3) | mant
    codes = np.where(sub, codes, norm).astype(np.int64)
    codes = np.where(y < 0, codes | 0x80, codes)
    codes = np.where(mag == 0, np.where(np.signbit(y), 0x80, 0), codes)
    return codes.astype(np.uint8)


def quantize_rows(x: np.ndarray):
    """(codes uint8 [rows][cols], exponents int32 [rows]) of x (fp32 math:
    x * 2^-e is exact; the value is clamped to +-448 before rounding)."""
    x = np.asarray(x, np.float32)
    e = row_exponents(x)
    y = np.ldexp(x.astype(np.float64), -e[:, None].astype(np.int64))
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    return encode(y), e


def dequantize_rows(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    return np.ldexp(VALUES[codes], e[:, None].astype(np.int64))


def quantize_kv(x: np.ndarray):
    """(codes uint8 [T][n_kv][hd], exponents int32 [T][n_kv]) of a K or V
    cache [T][n_kv][hd]: one row exponent per (token, KV head)."""
    T, H, D = x.shape
    c, e = quantize_rows(np.asarray(x, np.float32).reshape(T * H, D))
    return c.reshape(T, H, D), e.reshape(T, H)


def expand_kv(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    """The fp32 cache [T][n_kv][hd] that codes and exponents stand for:
    value(code) * 2^e, exact (an E4M3 value times a power of two is an fp32
    and a bf16 number)."""
    T, H, D = codes.shape
    return dequantize_rows(codes.reshape(T * H, D), e.reshape(T * H)).astype(np.float32).reshape(T, H, D)


def quantize_layer(w) -> dict:
    """8-bit weights of one layer: (codes, exponents) per projection matrix,
    quantized row by row (one exponent per output row)."""
    return {n: quantize_rows(w[n]) for n in ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down")}


def projector(w8: dict, act_store="bf16"):
    """Projections with 8-bit weights and activations, for oracle.layer's
    ``lin`` hook: the input rows are first rounded to the dtype they are
    stored in (the activations a projection reads are stored tensors), then
    quantized per row; the product of the decoded operands is exact in fp64
    and returned in fp32."""
    from .storage import round_store
    deq = {n: dequantize_rows(c, e) for n, (c, e) in w8.items()}

    def lin(x, name):
        xs = round_store(np.asarray(x, np.float32), act_store)
        c, e = quantize_rows(xs)
        return (dequantize_rows(c, e) @ deq[name].T).astype(np.float32)
    return lin


def gemm(a_codes, a_e, b_codes, b_e) -> np.ndarray:
    """C[m][n] = sum_k A[m][k] B[n][k] of the dequantized operands, in fp64."""
    return dequantize_rows(a_codes, a_e) @ dequantize_rows(b_codes, b_e).T
