"""The C-ABI library on the host: it loads, exports every call the header
declares, its host helpers agree with the oracle, and invalid arguments are
rejected with status codes before anything touches a device (CPU only)."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import blend, rope
from rag_kv_cache_layer_amd import fusor as F
from rag_kv_cache_layer_amd import synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "cacheblend.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cb_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(cblib):
    names = _declared()
    assert "cb_blend_layer" in names and "cb_rope_shift" in names and len(names) >= 12
    for n in names:
        assert hasattr(cblib, n), n


@pytest.mark.parametrize("theta,hd,n", [(1e4, 64, 300), (5e5, 128, 16448), (5e5, 64, 5000)])
def test_rope_table_bit_exact_vs_oracle(cblib, theta, hd, n):
    cfg = F.make_config(512, 8, 2, hd, 1024, theta, 1e-5, "bf16")
    c, s = F.rope_table(cfg, 0, n)
    oc, os_ = rope.rope_table(theta, hd, np.arange(n))
    assert np.array_equal(c.view(np.uint32), oc.view(np.uint32))
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32))
    c2, s2 = F.rope_table(cfg, 1000, 7)
    oc2, os2 = rope.rope_table(theta, hd, np.arange(1000, 1007))
    assert np.array_equal(c2, oc2) and np.array_equal(s2, os2)


def test_num_selected_and_schedule_match_oracle(cblib):
    for r in (0, 1, 500, 700, 1000, 1500, 3000, 10000):
        for n_ctx in (0, 1, 100, 128, 2048, 3072, 4000, 16384):
            for n_cand in (0, 50, n_ctx, n_ctx - 512 if n_ctx > 512 else 0):
                assert F.num_selected(r, n_ctx, n_cand) == blend.num_selected(r, n_ctx, n_cand), (r, n_ctx, n_cand)
    assert F.num_selected(700, 100, 100) == 7            # exact: no fp round-up
    assert F.num_selected(-1, 1, 1) == -1
    for L, a, b, n_ctx, n_cand in [(32, 3000, 1500, 4096, 3584), (80, 1500, 0, 4000, 3500), (2, 1500, 0, 3072, 2560),
                                   (5, 9000, 100, 1000, 300), (1, 1500, 0, 10, 5)]:
        assert F.filter_schedule(L, a, b, n_ctx, n_cand) == blend.filter_schedule(L, a, b, n_ctx, n_cand)


def test_status_strings(cblib):
    for s in range(7):
        assert F.status_string(s)
    assert F.status_string(99) == "unknown status"


def _cfg(**kw):
    base = dict(d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn_dim=1024, rope_theta=5e5, rms_eps=1e-5,
                dtype="bf16")
    base.update(kw)
    return F.make_config(**base)


def test_config_validation(cblib):
    assert F.workspace_size(_cfg(), 100, 100) > 0
    assert F.workspace_size(_cfg(n_q_heads=6, n_kv_heads=4), 100, 100) == 0     # heads not divisible
    assert F.workspace_size(_cfg(head_dim=96, n_q_heads=8, n_kv_heads=8), 10, 10) == 0  # bf16 hd 96
    assert F.workspace_size(_cfg(head_dim=96, n_q_heads=8, n_kv_heads=8, dtype="f32"), 10, 10) > 0
    assert F.workspace_size(_cfg(n_q_heads=24, n_kv_heads=2), 10, 10) == 0     # group of 12
    assert F.workspace_size(_cfg(d_model=500), 10, 10) == 0                     # d not a multiple of 8
    assert F.workspace_size(_cfg(ffn_dim=0), 10, 10) == 0
    # workspace grows with rows and covers the largest of T, m_max
    assert F.workspace_size(_cfg(), 200, 10) == F.workspace_size(_cfg(), 10, 200) > F.workspace_size(_cfg(), 10, 10)


FAKE = 1 << 20   # an aligned, never-dereferenced address: every case below fails before any device access


def _blend(L, cfg, **over):
    args = dict(w=F.LayerWeights(*([FAKE] * 9)), rope=F.rope_dev(cfg, FAKE, FAKE, 4096), k=FAKE, v=FAKE, T=100, n_ctx=90,
                L0=30, s_in=FAKE, m_in=70, h_in=FAKE, in_rows=None, k_out=9, h_out=FAKE, dev=None, s_out=FAKE,
                ws=FAKE, ws_bytes=1 << 40)
    args.update(over)
    m = ctypes.c_int32(-7)
    st = L.cb_blend_layer(ctypes.byref(cfg), ctypes.byref(args["w"]) if args["w"] is not None else None,
                          ctypes.byref(args["rope"]), args["k"], args["v"], args["T"], args["n_ctx"], args["L0"],
                          args["s_in"], args["m_in"], args["h_in"], args["in_rows"], args["k_out"], args["h_out"],
                          args["dev"], args["s_out"], ctypes.byref(m), args["ws"], args["ws_bytes"], None)
    return st, m.value


def test_blend_layer_argument_errors(cblib):
    L, cfg = cblib, _cfg()
    assert _blend(L, cfg, k=None)[0] == 1
    assert _blend(L, cfg, w=None)[0] == 1
    assert _blend(L, cfg, w=F.LayerWeights(*([FAKE] * 8 + [0])))[0] == 1          # null w_down
    assert _blend(L, cfg, h_in=FAKE + 2)[0] == 1                                   # misaligned
    assert _blend(L, cfg, k_out=-1)[0] == 1
    assert _blend(L, cfg, n_ctx=101)[0] == 2                                       # n_ctx > T
    assert _blend(L, cfg, L0=95)[0] == 2                                           # prefix past context
    assert _blend(L, cfg, m_in=5)[0] == 2                                          # misses query rows
    assert _blend(L, cfg, m_in=71)[0] == 2                                         # more rows than candidates
    assert _blend(L, cfg, rope=F.rope_dev(cfg, FAKE, FAKE, 99))[0] == 2                  # table too short
    assert _blend(L, cfg, ws_bytes=1000)[0] == 4
    assert _blend(L, _cfg(head_dim=96, n_q_heads=8, n_kv_heads=8))[0] == 5
    assert _blend(L, _cfg(dtype="f32"), T=9000, n_ctx=8990, rope=F.rope_dev(cfg, FAKE, FAKE, 9000))[0] == 5
    st, m = _blend(L, cfg, ws_bytes=1000)
    assert st == 4 and m == -7          # nothing written on failure before the size check
    st, m = _blend(L, cfg, m_in=10, k_out=3)   # all 10 rows are query rows: n_cand = 0 -> m_out = 10
    assert st != 1 and st != 2


def _realign(L, cfg, offs, n_chunks, **over):
    args = dict(w=F.LayerWeights(*([FAKE] * 9)), rope=F.rope_dev(cfg, FAKE, FAKE, 4096), k=FAKE, v=FAKE, T=100,
                s_in=FAKE, m_in=70, h_in=FAKE, in_rows=None, k_out=9, h_out=FAKE, dev=None, s_out=FAKE, ws=FAKE,
                ws_bytes=1 << 40)
    args.update(over)
    m = ctypes.c_int32(-7)
    st = L.cb_blend_layer_realign(ctypes.byref(cfg), ctypes.byref(args["w"]), ctypes.byref(args["rope"]),
                                  args["k"], args["v"], args["T"], offs, n_chunks, args["s_in"], args["m_in"],
                                  args["h_in"], args["in_rows"], args["k_out"], args["h_out"], args["dev"],
                                  args["s_out"], ctypes.byref(m), args["ws"], args["ws_bytes"], None)
    return st, m.value


def test_blend_layer_realign_argument_errors(cblib):
    """The offsets are checked as cb_rope_shift checks them, everything else
    as cb_blend_layer does (n_ctx and the first chunk come from the offsets)."""
    L, cfg = cblib, _cfg()
    offs = (ctypes.c_int32 * 4)(0, 30, 60, 90)
    assert _realign(L, cfg, None, 3)[0] == 1
    assert _realign(L, cfg, offs, 0)[0] == 1
    assert _realign(L, cfg, (ctypes.c_int32 * 4)(1, 30, 60, 90), 3)[0] == 2        # does not start at 0
    assert _realign(L, cfg, (ctypes.c_int32 * 4)(0, 60, 30, 90), 3)[0] == 2        # decreasing
    assert _realign(L, cfg, (ctypes.c_int32 * 4)(0, 30, 60, 101), 3)[0] == 2       # past T
    assert _realign(L, cfg, (ctypes.c_int32 * 258)(*range(258)), 257, T=300)[0] == 5
    assert _realign(L, cfg, offs, 3, k=None)[0] == 1
    assert _realign(L, cfg, offs, 3, m_in=5)[0] == 2          # misses query rows
    assert _realign(L, cfg, offs, 3, m_in=71)[0] == 2         # more rows than candidates after the first chunk
    assert _realign(L, cfg, offs, 3, rope=F.rope_dev(cfg, FAKE, FAKE, 99))[0] == 2
    assert _realign(L, cfg, offs, 3, rope=F.RopeDev(FAKE, FAKE, 4096, cfg.head_dim, 1e4))[0] == 1
    st, m = _realign(L, cfg, offs, 3, ws_bytes=1000)
    assert st == 4 and m == -7


def test_other_calls_argument_errors(cblib):
    L, cfg = cblib, _cfg()
    offs = (ctypes.c_int32 * 3)(0, 40, 90)
    rope_ok = F.rope_dev(cfg, FAKE, FAKE, 4096)
    assert L.cb_rope_shift(ctypes.byref(cfg), ctypes.byref(rope_ok), None, 0, 1, 100, offs, 2, None) == 1
    bad = (ctypes.c_int32 * 3)(0, 50, 40)
    assert L.cb_rope_shift(ctypes.byref(cfg), ctypes.byref(rope_ok), FAKE, 0, 1, 100, bad, 2, None) == 2
    over = (ctypes.c_int32 * 3)(0, 40, 101)
    assert L.cb_rope_shift(ctypes.byref(cfg), ctypes.byref(rope_ok), FAKE, 0, 1, 100, over, 2, None) == 2
    short = F.rope_dev(cfg, FAKE, FAKE, 40)
    assert L.cb_rope_shift(ctypes.byref(cfg), ctypes.byref(short), FAKE, 0, 1, 100, offs, 2, None) == 2
    assert L.cb_rope_shift(ctypes.byref(cfg), ctypes.byref(rope_ok), FAKE, 10, 2, 100, offs, 2, None) == 2
    many = (ctypes.c_int32 * 258)(*range(258))
    assert L.cb_rope_shift(ctypes.byref(cfg), ctypes.byref(rope_ok), FAKE, 0, 1, 300, many, 257, None) == 5
    # select: k > n, missing workspace
    assert L.cb_select_hkvd(ctypes.byref(cfg), None, None, 10, None, 5, 6, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert L.cb_select_hkvd(ctypes.byref(cfg), None, None, 10, None, 5, 2, FAKE, FAKE, None, 1 << 30, None) == 1
    assert L.cb_select_hkvd(ctypes.byref(cfg), None, None, 10, None, 5, 2, FAKE, FAKE, FAKE, 8, None) == 4
    # full prefill
    w = F.LayerWeights(*([FAKE] * 9))
    assert L.cb_full_prefill_layer(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(rope_ok), FAKE, 100, -1, FAKE,
                                   FAKE, FAKE, FAKE, 1 << 40, None) == 1
    assert L.cb_full_prefill_layer(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(short), FAKE, 100, 0, FAKE,
                                   FAKE, FAKE, FAKE, 1 << 40, None) == 2
    assert L.cb_full_prefill_layer(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(rope_ok), FAKE, 100, 0, FAKE,
                                   FAKE, FAKE, FAKE, 16, None) == 4
    # host helpers
    fp = ctypes.POINTER(ctypes.c_float)
    assert L.cb_rope_table(ctypes.byref(cfg), -1, 4, ctypes.cast(FAKE, fp), ctypes.cast(FAKE, fp)) == 1
    assert L.cb_filter_schedule(0, 1500, 0, 10, 5, None) == 1


def test_rope_table_must_match_config(cblib):
    """A device table built for another RoPE base or head size is refused by
    every call that reads one (it would rotate by the wrong angles)."""
    L, cfg = cblib, _cfg()
    offs = (ctypes.c_int32 * 3)(0, 40, 90)
    w = F.LayerWeights(*([FAKE] * 9))
    good = F.rope_dev(cfg, FAKE, FAKE, 4096)
    other_base = F.RopeDev(FAKE, FAKE, 4096, cfg.head_dim, 1e4)
    other_hd = F.RopeDev(FAKE, FAKE, 4096, 128, cfg.rope_theta)
    for bad in (other_base, other_hd):
        assert L.cb_rope_shift(ctypes.byref(cfg), ctypes.byref(bad), FAKE, 0, 1, 100, offs, 2, None) == 1
        assert _blend(L, cfg, rope=bad)[0] == 1
        assert L.cb_full_prefill_layer(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(bad), FAKE, 100, 0, FAKE,
                                       FAKE, FAKE, FAKE, 1 << 40, None) == 1
        assert L.cb_kv_from_fp8(ctypes.byref(cfg), ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, 1, 0, 100, FAKE, FAKE,
                                0, 100, offs, 2, 1, None) == 1
    # tables must be 16-byte aligned
    misaligned = F.RopeDev(FAKE + 4, FAKE, 4096, cfg.head_dim, cfg.rope_theta)
    assert _blend(L, cfg, rope=misaligned)[0] == 1
    assert L.cb_rope_shift(ctypes.byref(cfg), ctypes.byref(misaligned), FAKE, 0, 1, 100, offs, 2, None) == 1
    # the same table with matching fields passes the check (and fails later, on the workspace)
    assert L.cb_full_prefill_layer(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(good), FAKE, 100, 0, FAKE,
                                   FAKE, FAKE, FAKE, 16, None) == 4


def test_profile_without_launches(cblib):
    F.profile_begin()
    assert F.profile_end() == {}


def test_8bit_calls_argument_errors(cblib):
    L, cfg = cblib, _cfg()
    rope_ok = F.rope_dev(cfg, FAKE, FAKE, 4096)
    w8 = F.LayerWeightsFp8(*([FAKE] * 10))
    m = ctypes.c_int32(-7)

    def blend8(c=cfg, w=w8, ws_bytes=1 << 40):
        return L.cb_blend_layer_fp8(ctypes.byref(c), ctypes.byref(w) if w is not None else None,
                                    ctypes.byref(rope_ok), FAKE, FAKE, 100, 90, 30, FAKE, 70, FAKE, None, 9, FAKE,
                                    None, FAKE, ctypes.byref(m), FAKE, ws_bytes, None)
    assert blend8(w=None) == 1
    assert blend8(w=F.LayerWeightsFp8(*([FAKE] * 9 + [0]))) == 1                  # null e_down
    assert blend8(w=F.LayerWeightsFp8(FAKE, FAKE + 8, *([FAKE] * 8))) == 1        # misaligned codes
    assert blend8(c=_cfg(dtype="f32")) == 5
    assert blend8(c=_cfg(d_model=520)) == 2                                        # d not a multiple of 16
    assert blend8(ws_bytes=1000) == 4
    assert m.value == -7
    assert int(L.cb_workspace_size_fp8(ctypes.byref(cfg), 100, 100)) > F.workspace_size(cfg, 100, 100)
    offs = (ctypes.c_int32 * 3)(0, 40, 90)
    kv = L.cb_kv_from_fp8
    assert kv(ctypes.byref(cfg), ctypes.byref(rope_ok), None, FAKE, FAKE, FAKE, 1, 0, 100, FAKE, FAKE, 0, 100, offs,
              2, 1, None) == 1
    assert kv(ctypes.byref(cfg), ctypes.byref(rope_ok), FAKE + 4, FAKE, FAKE, FAKE, 1, 0, 100, FAKE, FAKE, 0, 100,
              offs, 2, 1, None) == 1                                               # misaligned codes
    assert kv(ctypes.byref(cfg), ctypes.byref(rope_ok), FAKE, FAKE, FAKE, FAKE, 1, 50, 51, FAKE, FAKE, 0, 100, offs,
              2, 1, None) == 2                                                     # rows past T
    short = F.rope_dev(cfg, FAKE, FAKE, 40)
    assert kv(ctypes.byref(cfg), ctypes.byref(short), FAKE, FAKE, FAKE, FAKE, 1, 0, 100, FAKE, FAKE, 0, 100, offs,
              2, 1, None) == 2                                                     # table too short for the shift
    cf72 = _cfg(dtype="f32", head_dim=72, n_q_heads=8, n_kv_heads=8, d_model=576)
    assert F.workspace_size(cf72, 10, 10) > 0
    assert kv(ctypes.byref(cf72), ctypes.byref(F.rope_dev(cf72, FAKE, FAKE, 4096)), FAKE, FAKE, FAKE, FAKE, 1, 0, 100, FAKE, FAKE, 0, 100,
              offs, 2, 1, None) == 2                                               # head_dim not a multiple of 16
    many = (ctypes.c_int32 * 258)(*range(258))
    assert kv(ctypes.byref(cfg), ctypes.byref(rope_ok), FAKE, FAKE, FAKE, FAKE, 1, 0, 100, FAKE, FAKE, 0, 300, many,
              257, 1, None) == 5
    # nothing to expand: no device access at all
    assert kv(ctypes.byref(cfg), None, FAKE, FAKE, FAKE, FAKE, 1, 0, 0, FAKE, FAKE, 0, 100, offs, 2, 0, None) == 0
    assert kv(ctypes.byref(cfg), None, FAKE, FAKE, FAKE, FAKE, 0, 0, 100, FAKE, FAKE, 0, 100, offs, 2, 0, None) == 0
    # the 8-bit stack needs all four sources
    ks = (ctypes.c_int32 * 2)(10, 10)
    Wl = (F.LayerWeights * 2)(F.LayerWeights(*([FAKE] * 9)), F.LayerWeights(*([FAKE] * 9)))
    assert L.cb_blend_stack_kv8(ctypes.byref(cfg), 2, Wl, ctypes.byref(rope_ok), FAKE, FAKE, 100 * 128, FAKE, None,
                                FAKE, FAKE, 100, offs, 2, 1, FAKE, ks, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None,
                                None) == 1


def test_gemm_fp8_noalloc_argument_errors(cblib):
    L = cblib
    g = lambda M, N, K, a=FAKE, ldc=None, od=0: L.cb_gemm_fp8_noalloc(M, N, K, a, FAKE, FAKE, FAKE, FAKE,
                                                                        N if ldc is None else ldc, od, None)
    assert g(-1, 16, 16) == 1
    assert g(4, 16, 16, ldc=8) == 1
    assert g(4, 16, 16, od=7) == 1
    assert g(4, 16, 16, a=None) == 1
    assert g(4, 16, 24) == 2                                   # K not a multiple of 16
    assert g(4, 16, 16, a=FAKE + 4) == 2                       # misaligned codes
    assert g(0, 16, 16) == 0                                   # nothing to do
    # split-K partials beyond the static array: 2 x 1100 x 4096 x 4 B > 32 MiB
    assert int(L.cb_gemm_fp8_workspace_size(1100, 4096, 4096)) > F.GEMM_FP8_SCRATCH_BYTES
    assert g(1100, 4096, 4096) == 4


def test_analytics_argument_errors(cblib):
    L, cfg = cblib, _cfg()
    assert int(L.cb_workspace_q_offset(ctypes.byref(cfg), 100)) > 0
    assert int(L.cb_workspace_q_offset(ctypes.byref(cfg), 0)) == 0
    assert int(L.cb_workspace_q_offset(ctypes.byref(_cfg(n_q_heads=6, n_kv_heads=4)), 100)) == 0
    need = int(L.cb_analytics_workspace_size(10, 8, 0))
    assert need >= 10 * 8 * 2 * 8
    ad = L.cb_attention_deviation
    assert ad(ctypes.byref(cfg), -1, FAKE, FAKE, FAKE, FAKE, 100, FAKE, FAKE, FAKE, need, None) == 1
    assert ad(ctypes.byref(cfg), 10, FAKE, None, FAKE, FAKE, 100, FAKE, FAKE, FAKE, need, None) == 1
    assert ad(ctypes.byref(cfg), 10, FAKE, FAKE, FAKE, FAKE, 100, FAKE, FAKE, FAKE, need - 1, None) == 4
    assert ad(ctypes.byref(cfg), 0, None, None, None, None, 100, None, FAKE, None, 0, None) == 0
    n_need = int(L.cb_analytics_workspace_size(0, 0, 50))
    assert L.cb_spearman(FAKE, FAKE, 0, FAKE, FAKE, n_need, None) == 1
    assert L.cb_spearman(FAKE, FAKE, 50, FAKE, FAKE, n_need - 1, None) == 4
    assert L.cb_top_share(FAKE, 50, 51, FAKE, FAKE, n_need, None) == 1
    assert L.cb_top_share(FAKE, 50, 5, FAKE, FAKE, n_need - 1, None) == 4


def test_validate_switch(cblib):
    assert F.set_validate(True) is False
    assert F.set_validate(False) is True
    assert F.set_validate(False) is False


def test_pack_gateup_argument_errors(cblib):
    L, cfg = cblib, _cfg()
    assert int(L.cb_pack_gateup_size(ctypes.byref(cfg))) == 10 * 16 * 224 * 64  # ceil(1024/112) tiles x 512/32 steps
    assert int(L.cb_pack_gateup_size(ctypes.byref(_cfg(dtype="f32")))) == 0
    assert L.cb_pack_gateup(ctypes.byref(_cfg(dtype="f32")), FAKE, FAKE, FAKE, None) == 5
    assert L.cb_pack_gateup(ctypes.byref(cfg), None, FAKE, FAKE, None) == 1
    assert L.cb_pack_gateup(ctypes.byref(cfg), FAKE, FAKE, FAKE + 4, None) == 1
    w = F.LayerWeights(*([FAKE] * 9 + [FAKE + 2]))                               # misaligned packed copy
    assert _blend(L, cfg, w=w)[0] == 1


def test_fold_qkv_argument_errors(cblib):
    L, cfg = cblib, _cfg()
    # [W_q; W_k; W_v] rows x d_model bf16
    assert int(L.cb_fold_qkv_size(ctypes.byref(cfg))) == (512 + 2 * 128) * 512 * 2
    assert int(L.cb_fold_qkv_size(ctypes.byref(_cfg(dtype="f32")))) == 0
    w = F.LayerWeights(*([FAKE] * 9))
    assert L.cb_fold_qkv(ctypes.byref(_cfg(dtype="f32")), ctypes.byref(w), FAKE, None) == 5
    assert L.cb_fold_qkv(ctypes.byref(cfg), None, FAKE, None) == 1
    assert L.cb_fold_qkv(ctypes.byref(cfg), ctypes.byref(w), FAKE + 8, None) == 1
    assert L.cb_fold_qkv(ctypes.byref(cfg), ctypes.byref(F.LayerWeights(*([FAKE] * 3))), FAKE, None) == 1
    wf = F.LayerWeights(*([FAKE] * 10 + [FAKE + 4]))                             # misaligned folded copy
    assert _blend(L, cfg, w=wf)[0] == 1
