"""cb_gemm_fp8_noalloc, the 8-bit GEMM whose split-K partials live in the
library's static per-GPU array instead of a caller workspace, against
cb_gemm_fp8 with a workspace (the same kernels, so the same bits) and the
oracle's exact product.  Two calls in a row on the same GPU, the second with
a smaller input, so the second reads an array still holding the first
call's partials; then a shape without split-K, and a call whose partials
would not fit, which is refused before any device work."""
import numpy as np
import pytest

from oracle import fp8
from rag_kv_cache_layer_amd import fusor as F
from tests.gpu_util import need_gpu, rel_err, torch

pytestmark = pytest.mark.gpu


def _operands(rng, M, N, K):
    a = (rng.normal(size=(M, K)) * np.exp(rng.uniform(-4, 4, (M, 1)))).astype(np.float32)
    b = (rng.normal(size=(N, K)) * 0.02).astype(np.float32)
    ac, ae = fp8.quantize_rows(a)
    bc, be = fp8.quantize_rows(b)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return (ac, ae, bc, be), [dev(x) for x in (ac, ae, bc, be)]


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_equals_workspace_call_twice(out_dtype):
    need_gpu()
    rng = np.random.default_rng(5)
    shapes = [(493, 4096, 4096), (130, 4096, 14336), (77, 6144, 4096)]
    for M, N, K in shapes:
        host_ops, (a, ae, b, be) = _operands(rng, M, N, K)
        need = int(F.lib().cb_gemm_fp8_workspace_size(M, N, K))
        assert need <= F.GEMM_FP8_SCRATCH_BYTES
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        ref = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
        got = torch.full((M, N), float("nan"), dtype=out_dtype, device="cuda")
        F.gemm_fp8(a, ae, b, be, ref, ws=ws)
        F.gemm_fp8_noalloc(a, ae, b, be, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), (M, N, K)
        if out_dtype == torch.float32:
            want = fp8.gemm(*host_ops)
            assert rel_err(got.cpu().numpy(), want) < 1e-4, (M, N, K)


def test_noalloc_refuses_partials_beyond_the_array():
    need_gpu()
    M, N, K = 1100, 4096, 4096          # 2 splits x 1100 x 4096 x 4 B = 36 MB > 32 MiB
    assert int(F.lib().cb_gemm_fp8_workspace_size(M, N, K)) > F.GEMM_FP8_SCRATCH_BYTES
    a = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
    b = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
    ae = torch.zeros(M, dtype=torch.int32, device="cuda")
    be = torch.zeros(N, dtype=torch.int32, device="cuda")
    out = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(F.CacheBlendError) as e:
        F.gemm_fp8_noalloc(a, ae, b, be, out)
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
