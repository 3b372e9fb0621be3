"""8-bit float operands (OCP E4M3, one power-of-two scale per row) on the GPU
against the oracle (oracle/fp8.py).

* Quantization: codes and row exponents bit for bit, from bf16 and fp32
  inputs, on random rows of very different magnitudes and on edge rows (all
  zero, a single nonzero, values exactly at 448 * 2^k and just above, values
  that fall below the smallest subnormal, ties).  The rounding decision is an
  integer result taken in the same precision on both sides.
* GEMM: fp32 output within 1e-4 of the oracle's fp64 sum of the decoded
  products (per tensor, max |x - y| / max |y|), ragged tiles, the split-K path,
  the 256x256 kernel for wide outputs (ragged rows, columns and K; vector and
  element stores) and the 8B layer's projection shapes (rows sampled); bf16
  output within bf16 rounding.  Every product of two E4M3 values is exact, but the matrix
  core adds the products of a 128-long block at a precision below fp32 (the
  measured difference from an exact sum is about 1e-5 of the largest
  output), hence 1e-4 rather than fp32 rounding; it is still 500x below the
  E4M3 quantization error of 2^-4."""
import numpy as np
import pytest

from oracle import fp8
from rag_kv_cache_layer_amd import fusor as F
from tests.gpu_util import need_gpu, rel_err, torch

pytestmark = pytest.mark.gpu


def _rows(rng, rows, cols):
    x = rng.normal(size=(rows, cols)) * np.exp(rng.uniform(-12, 12, (rows, 1)))
    x[0] = 0.0
    if rows > 3:
        x[1] = 0.0
        x[1, cols // 2] = -3.5
        x[2] = rng.normal(size=cols) * 1e-3
        x[2, 0] = 448.0 * 2.0 ** -4                 # amax exactly 448 * 2^-4
        x[3] = 1e-30                                 # everything below the fp8 grid after scaling
        x[3, -1] = 1.0
    return x.astype(np.float32)


@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(1, 16), (7, 33), (64, 4096), (300, 1000)])
def test_quantize_bit_exact(src, shape):
    need_gpu()
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    x = _rows(rng, *shape)
    if src == "bf16":
        xt = torch.from_numpy(x).cuda().to(torch.bfloat16)
        xh = xt.float().cpu().numpy()
    else:
        xt = torch.from_numpy(x).cuda()
        xh = x
    codes, exps = F.quantize_fp8(xt)
    torch.cuda.synchronize()
    wc, we = fp8.quantize_rows(xh)
    assert np.array_equal(exps.cpu().numpy(), we)
    got = codes.cpu().numpy()
    # -0 and +0 decode alike; compare codes with zeros folded
    fold = lambda c: np.where((c & 0x7F) == 0, 0, c)
    assert np.array_equal(fold(got), fold(wc))


@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (37, 200, 528), (130, 257, 4096), (200, 128, 1024),
                                   (300, 24584, 528), (257, 24653, 400)])
def test_gemm_matches_oracle(M, N, K):
    need_gpu()
    rng = np.random.default_rng(M + N + K)
    a = rng.normal(size=(M, K)).astype(np.float32)
    b = (rng.normal(size=(N, K)) * 0.02).astype(np.float32)
    qa, ea = fp8.quantize_rows(a)
    qb, eb = fp8.quantize_rows(b)
    want = fp8.gemm(qa, ea, qb, eb)
    ta = torch.from_numpy(qa).cuda()
    tb = torch.from_numpy(qb).cuda()
    tea, teb = torch.from_numpy(ea).cuda(), torch.from_numpy(eb).cuda()
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    F.gemm_fp8(ta, tea, tb, teb, out)
    out16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    F.gemm_fp8(ta, tea, tb, teb, out16)
    torch.cuda.synchronize()
    e32 = rel_err(out.cpu().numpy(), want)
    print(f"\nM={M} N={N} K={K}: fp32 output max-rel error {e32:.3g}")
    assert e32 < 1e-4
    assert rel_err(out16.float().cpu().numpy(), want) < 2 ** -8


@pytest.mark.parametrize("N,K", [(6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336)])
def test_gemm_layer_shapes_sampled(N, K):
    """The 8B layer's projections at 493 rows: full-size launch, 24 rows
    checked against the oracle."""
    need_gpu()
    M = 493
    g = torch.Generator(device="cuda")
    g.manual_seed(N + K)
    a = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    b = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    qa, ea = F.quantize_fp8(a)
    qb, eb = F.quantize_fp8(b)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    F.gemm_fp8(qa, ea, qb, eb, out)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(M, 24, replace=False)
    rows = np.unique(np.concatenate([rows, [0, M - 1]]))
    qa_h, ea_h = qa.cpu().numpy()[rows], ea.cpu().numpy()[rows]
    want = fp8.gemm(qa_h, ea_h, qb.cpu().numpy(), eb.cpu().numpy())
    e32 = rel_err(out.cpu().numpy()[rows], want)
    print(f"\nM={M} N={N} K={K}: fp32 output max-rel error {e32:.3g}")
    assert e32 < 1e-4
    # the quantizer matched the oracle on these inputs too
    wq, we = fp8.quantize_rows(a.float().cpu().numpy()[rows])
    assert np.array_equal(ea_h, we)
