"""The loading controller and the stack entry point on the host (CPU only).

cb_pick_ratio follows CacheBlend section 5 (loading controller): the
recompute delay of ratio r is r times an offline-profiled full prefill of the
layer (footnote 5), the load delay is KV bytes per token times tokens over the
device throughput (footnote 6); the ratio that makes the two equal is taken,
then raised to the quality floor r* = 15% (Figure 16).  The pins are the
pages' own numbers: the explainer's example of an SSD that loads a layer in
16 ms while the 15% recompute takes 3 ms (so a full prefill takes 20 ms and the
matching ratio is 16/20 = 80%), and CPU RAM loading a layer in about 1 ms,
where the floor decides.  cb_blend_stack must reject bad arguments before it
touches a device."""
import ctypes

import numpy as np
import pytest

from rag_kv_cache_layer_amd import fusor as F

KV_TOKEN = 8 * 128 * 2 * 2     # bytes of one layer's K and V per token, 8 KV heads of 128, bf16


def test_ratio_matches_the_explainers_ssd_example(cblib):
    # T_recompute(15%) = 3 ms  =>  T_prefill = 20 ms; T_load = 16 ms
    n = 4000
    link = KV_TOKEN * n / 16000.0            # bytes per microsecond giving a 16 ms load
    assert F.pick_ratio(20000.0, KV_TOKEN, n, link, 1500) == 8000
    # recompute at that ratio equals the load time
    assert abs(0.8 * 20000.0 - KV_TOKEN * n / link) < 1e-9


def test_fast_storage_is_floored_at_the_quality_minimum(cblib):
    n = 4000
    link = KV_TOKEN * n / 1000.0             # CPU RAM: about 1 ms per layer
    assert F.pick_ratio(20000.0, KV_TOKEN, n, link, 1500) == 1500      # r_match = 5% < 15%
    assert F.pick_ratio(20000.0, KV_TOKEN, n, link, 0) == 500
    assert F.pick_ratio(20000.0, KV_TOKEN, n, link, 300) == 500


def test_ratio_rounds_down_caps_and_is_monotone(cblib):
    # r_match = 1/3 -> 3333 (never rounds up past the load time)
    assert F.pick_ratio(3000.0, 1.0, 1000, 1.0, 0) == 3333
    # slower link or longer context -> larger ratio, capped at 1
    prev = -1
    for link in (1e6, 1e5, 1e4, 1e3, 1e2, 1e1):
        r = F.pick_ratio(1000.0, KV_TOKEN, 4000, link, 0)
        assert r >= prev
        prev = r
    assert prev == 10000
    assert F.pick_ratio(1.0, 1e9, 10, 1.0, 1500) == 10000


@pytest.mark.parametrize("args", [(0.0, 1.0, 1, 1.0, 0), (-1.0, 1.0, 1, 1.0, 0), (1.0, 0.0, 1, 1.0, 0),
                                  (1.0, 1.0, 0, 1.0, 0), (1.0, 1.0, 1, 0.0, 0), (1.0, 1.0, 1, 1.0, -1),
                                  (1.0, 1.0, 1, 1.0, 10001), (float("inf"), 1.0, 1, 1.0, 0),
                                  (float("nan"), 1.0, 1, 1.0, 0)])
def test_ratio_rejects_invalid_inputs(cblib, args):
    assert cblib.cb_pick_ratio(*args) == -1


def test_stack_workspace_covers_a_layer_and_two_hidden_buffers(cblib):
    cfg = F.make_config(4096, 32, 8, 128, 14336, 5e5, 1e-5, "bf16")
    T = 4160
    n = F.stack_workspace_size(cfg, T)
    assert n >= F.workspace_size(cfg, T, T) + 2 * T * 4096 * 2 + T * 4
    assert F.stack_workspace_size(cfg, 0) == 0


def test_stack_rows_follow_the_schedule(cblib):
    offs = [0, 512, 1024, 1536, 2048, 2560, 3072]
    m_in, m_out = F.stack_rows(3104, offs, [461, 461, 300, 0])
    assert m_in == [2592, 493, 493, 332] and m_out == [493, 493, 332, 32]
    m_in, m_out = F.stack_rows(200, [0, 200], [5, 5])   # one chunk: only the query rows
    assert m_in == [0, 0] and m_out == [0, 0]


def _fake(n, align=256):
    """Non-null, aligned host addresses that the checks accept as pointers
    (the calls below must fail before they are used)."""
    return ctypes.c_void_p(0x10000 + n * align)


def test_stack_rejects_bad_arguments_before_any_device_work(cblib):
    cfg = F.make_config(256, 4, 4, 64, 688, 1e4, 1e-5, "bf16")
    T = 144
    w = F.LayerWeights(*[0x20000 + 256 * i for i in range(9)])
    W = (F.LayerWeights * 2)(w, w)
    rope = F.rope_dev(cfg, 0x30000, 0x40000, T)
    offs = np.array([0, 64, 128], dtype=np.int32)
    ks = np.array([20, 20], dtype=np.int32)
    I32P = ctypes.POINTER(ctypes.c_int32)
    need = F.stack_workspace_size(cfg, T)

    def call(k_src=None, v_src=None, ws_bytes=need, ks_=ks, n_layers=2, stride=T * 256, rope_=rope):
        return cblib.cb_blend_stack(ctypes.byref(cfg), n_layers, W, ctypes.byref(rope_), _fake(1), _fake(2), stride,
                                    k_src, v_src, T, offs.ctypes.data_as(I32P), 2, 1, _fake(3),
                                    ks_.ctypes.data_as(I32P), _fake(4), _fake(5), _fake(6), None, _fake(7),
                                    ws_bytes, None, None)

    assert call(k_src=_fake(8)) == 1                          # k_src without v_src
    assert call(ws_bytes=need - 1) == 4                       # CB_ERR_WORKSPACE
    assert call(ks_=np.array([20, -1], dtype=np.int32)) == 1  # negative k_out
    assert call(n_layers=0) == 1
    assert call(stride=T * 256 - 8) == 2                      # layers overlap
    assert call(rope_=F.rope_dev(cfg, 0x30000, 0x40000, T - 1)) == 2


def test_batch_rejects_bad_arguments_before_any_device_work(cblib):
    cfg = F.make_config(256, 4, 4, 64, 688, 1e4, 1e-5, "bf16")
    w = F.LayerWeights(*[0x20000 + 256 * i for i in range(9)])
    rope = F.rope_dev(cfg, 0x30000, 0x40000, 200)

    def req(T=144, n_ctx=128, L0=64, m_in=36, k=20, kc=0x50000):
        return F.BlendRequest(kc, kc + 0x100000, T, n_ctx, L0, m_in, k)

    def call(reqs, ws_bytes=1 << 40):
        arr = (F.BlendRequest * max(len(reqs), 1))(*reqs)
        return cblib.cb_blend_batch(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(rope), len(reqs), arr,
                                    _fake(1), _fake(2), _fake(3), None, _fake(4), None, _fake(5), ws_bytes, None)

    assert call([]) == 1                                  # no request
    assert call([req()] * 17) == 5                        # more than 16 requests
    assert call([req(), req(n_ctx=150)]) == 2             # n_ctx > T
    assert call([req(), req(m_in=100)]) == 2              # more candidates than rows past the prefix
    assert call([req(), req(m_in=10)]) == 2               # fewer rows than query rows
    assert call([req(), req(kc=0x50008)]) == 1            # misaligned cache
    assert call([req(), req(T=300, n_ctx=284, m_in=36)]) == 2   # rope table shorter than T
    need = F.workspace_size(cfg, 144, 72)
    assert call([req(), req()], need - 1) == 4
