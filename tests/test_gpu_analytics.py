"""Deviation analytics on the GPU (CacheBlend sections 4.1-4.3, Figures 6-8).

* The library's statistics equal the oracle's (numpy, fp64) on the same
  seeded data: the attention deviation and the squared norm of the reference
  attention matrix (GQA, ragged causal limits, fp32 and bf16 operands)
  within fp32 rounding of the probabilities; Spearman's correlation with
  ties and the top shares to fp64 rounding.
* A reduced 4-layer stack through the library: at r = 1 the blended run
  reproduces full prefill, so its attention deviation is rounding only and
  smaller than at r = 0; deviations and correlations are finite and in
  range; the per-layer lists have the stack's length.  How the deviation
  falls between the end points with random weights is reported, not gated
  (random weights need not have the sparsity of trained ones)."""
import math

import numpy as np
import pytest

from oracle import analytics as OA
from rag_kv_cache_layer_amd import analytics as GA
from rag_kv_cache_layer_amd import fusor as F
from rag_kv_cache_layer_amd import synth
from tests.gpu_util import need_gpu, torch


pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,hd,n_q,n_kv,T", [("f32", 16, 8, 2, 40), ("bf16", 128, 32, 8, 300),
                                                 ("f32", 72, 6, 3, 700)])
def test_attention_deviation_matches_oracle(dtype, hd, n_q, n_kv, T):
    need_gpu()
    rng = np.random.default_rng(hd + T)
    m = 9
    cfg = F.make_config(n_q * hd, n_q, n_kv, hd, 256, 5e5, 1e-5, dtype)
    r = (lambda x: synth.round_to(x, dtype))
    qa = r(rng.normal(size=(m, n_q, hd)).astype(np.float32) * 0.5)
    qb = r(qa + rng.normal(size=qa.shape).astype(np.float32) * 0.2)
    ka = r(rng.normal(size=(T, n_kv, hd)).astype(np.float32))
    kb = r(ka + rng.normal(size=ka.shape).astype(np.float32) * 0.1)
    last = np.sort(rng.integers(0, T, m)).astype(np.int32)
    last[0], last[-1] = 0, T - 1
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(dt)
    d2, n2 = F.attention_deviation(cfg, dev(qa), dev(ka), dev(qb), dev(kb), torch.from_numpy(last).cuda())
    Aa = OA.attention_matrix(qa, ka, last)
    Ab = OA.attention_matrix(qb, kb, last)
    want_d = OA.attention_deviation(Aa, Ab)
    want_n = OA.attention_deviation(Ab, np.zeros_like(Ab))
    assert abs(math.sqrt(d2) - want_d) <= 1e-5 * want_n + 1e-6 * want_d, (math.sqrt(d2), want_d)
    assert abs(math.sqrt(n2) - want_n) <= 1e-5 * want_n, (math.sqrt(n2), want_n)
    # identical matrices: exactly zero
    d0, _ = F.attention_deviation(cfg, dev(qa), dev(ka), dev(qa), dev(ka), torch.from_numpy(last).cuda())
    assert d0 == 0.0


@pytest.mark.parametrize("n", [3, 50, 2560, 15872])
def test_rank_statistics_match_oracle(n):
    need_gpu()
    rng = np.random.default_rng(n)
    x = rng.integers(0, 9, n).astype(np.float32)            # many ties
    y = (x + rng.normal(0, 3, n)).astype(np.float32)
    got, want = F.spearman(torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()), OA.spearman(x, y)
    assert (math.isnan(got) and math.isnan(want)) or abs(got - want) < 1e-12
    z = rng.normal(size=n).astype(np.float32)
    assert abs(F.spearman(torch.from_numpy(z).cuda(), torch.from_numpy(-z).cuda()) + 1.0) < 1e-12
    d = rng.exponential(size=n).astype(np.float32)
    d[: n // 3] = d[0]                                       # ties at the boundary
    for f in (0.1, 0.15, 0.2, 1.0):
        k = int(math.ceil(f * n - 1e-9))
        assert abs(F.top_share(torch.from_numpy(d).cuda(), k) - OA.top_share(d, f)) < 1e-12


def test_stack_study_endpoints():
    need_gpu()
    p = synth.scaled(synth.PRESETS["llama8b_stack"], 512, 8, 2, 64, 1024, [60, 45, 70, 33], 7, n_layers=4)
    cfg = F.config_of(p)
    ws_ = [synth.layer_weights(p, 31, l) for l in range(p.n_layers)]
    layers = [F.DeviceLayer(cfg, w) for w in ws_]
    rope = F.DeviceRope(cfg, p.T)
    order = synth.chunk_order(p, 31)
    offs = synth.chunk_offsets(p, order)
    x_all = torch.from_numpy(synth.context_embeddings(p, 31, order)).cuda().to(torch.bfloat16)
    out = GA.stack_study(cfg, layers, rope, x_all, offs, [0, 1500, 10000])
    d0, d15, d1 = out["attn_dev_mean"]
    print(f"\nattention deviation (relative, mean over layers): r=0 {d0:.4g}, r=0.15 {d15:.4g}, r=1 {d1:.4g}; "
          f"spearman {['%.3f' % s for s in out['spearman_neighbours']]}, top15 {out['top_share']['0.15']}")
    assert all(len(x) == p.n_layers for x in out["attn_dev"])
    assert d1 < 2e-2 and d1 < d0
    assert all(-1.0 <= s <= 1.0 for s in out["spearman_neighbours"])
    for f, shares in out["top_share"].items():
        assert all(float(f) - 1e-6 <= s <= 1.0 for s in shares)   # the top f hold at least f of the total
