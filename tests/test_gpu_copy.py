"""cb_stream_copy, the streaming copy the bandwidth-bound kernels are
measured against: a byte-exact copy for sizes that fill whole blocks, end in
a ragged block, or hold a single 16-byte unit, leaving the bytes after the
range untouched."""
import pytest

from rag_kv_cache_layer_amd import fusor as F
from tests.gpu_util import need_gpu, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 4, 4096 * 4 + 48, 3 * 1000 * 1000 - 16 * 7, 64 << 20])
def test_stream_copy_exact(nbytes):
    need_gpu()
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.full((nbytes + 64,), 7, dtype=torch.uint8, device="cuda")
    F.stream_copy(src, dst[:nbytes])
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 7).all())
