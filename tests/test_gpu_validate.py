"""Validate mode (cb_set_validate): the index arrays the calls read from the
device are checked on the host first.  Invalid rows give CB_ERR_INDEX (3) and
a NaN in a deviation array given as input CB_ERR_ARG (1), with nothing
enqueued (the outputs keep their sentinels); valid inputs give the same bits
as without validation.  Every invalid case is rejected on the host, so no
kernel ever sees it."""
import numpy as np
import pytest

from rag_kv_cache_layer_amd import fusor as F
from rag_kv_cache_layer_amd import synth
from tests.gpu_util import dev, host, need_gpu, single_layer_case, torch

pytestmark = pytest.mark.gpu

P = synth.scaled(synth.PRESETS["llama8b_layer"], 512, 8, 2, 64, 1024, [90, 61, 120], 9)


@pytest.fixture
def validating():
    prev = F.set_validate(True)
    yield
    F.set_validate(prev)


def _setup():
    case = single_layer_case(P, 0, prepass_inputs=False)
    cfg = F.config_of(P)
    return case, cfg, F.DeviceLayer(cfg, case["w"]), F.DeviceRope(cfg, P.T), F.workspace(cfg, P.T, P.T)


def _call(cfg, layer, rope, ws, case, s_in, in_rows, k):
    T, n_ctx, L0 = P.T, P.n_ctx, case["L0"]
    kc, vc = dev(case["k"], torch.bfloat16), dev(case["v"], torch.bfloat16)
    m_in = len(s_in)
    hout = torch.full((m_in, P.d_model), 7.0, dtype=torch.bfloat16, device="cuda")
    dv = torch.full((m_in,), 7.0, dtype=torch.float32, device="cuda")
    so = torch.full((m_in,), -5, dtype=torch.int32, device="cuda")
    s_t = dev(np.asarray(s_in, np.int32), torch.int32)
    r_t = None if in_rows is None else dev(np.asarray(in_rows, np.int32), torch.int32)
    hid = dev(case["hidden"], torch.bfloat16)
    try:
        F.blend_layer(cfg, layer, rope, kc, vc, T, n_ctx, L0, s_t, m_in, hid, r_t if r_t is not None else s_t, k,
                      hout, dv, so, ws)
        st = 0
    except F.CacheBlendError as e:
        st = e.status
    torch.cuda.synchronize()
    return st, dict(k=host(kc), v=host(vc), y=host(hout), dev=host(dv), s_out=so.cpu().numpy())


def test_blend_layer_index_validation(validating):
    need_gpu()
    case, cfg, layer, rope, ws = _setup()
    T, n_ctx, L0 = P.T, P.n_ctx, case["L0"]
    s_all = np.arange(L0, T)
    k = 20
    bad = []
    b = s_all.copy(); b[[3, 4]] = b[[4, 3]]; bad.append((b, None))          # not ascending
    b = s_all.copy(); b[0] = L0 - 1; bad.append((b, None))                  # a prefix row
    b = s_all.copy(); b[-1] = T; bad.append((b, None))                      # past T
    r = s_all.copy(); r[5] = T + 3; bad.append((s_all, r))                   # in_rows past T
    r = s_all.copy(); r[0] = -1; bad.append((s_all, r))                      # negative in_rows
    for s_in, rows in bad:
        st, out = _call(cfg, layer, rope, ws, case, s_in, rows, k)
        assert st == 3, (s_in[:5], s_in[-5:])
        assert np.all(out["y"] == 7.0) and np.all(out["dev"] == 7.0) and np.all(out["s_out"] == -5)
        assert np.array_equal(out["k"], case["k"])
    # a valid call: the same bits as without validation
    st, got = _call(cfg, layer, rope, ws, case, s_all, None, k)
    assert st == 0
    F.set_validate(False)
    st2, ref = _call(cfg, layer, rope, ws, case, s_all, None, k)
    F.set_validate(True)
    assert st2 == 0
    for key in ("k", "v", "y", "s_out"):
        assert np.array_equal(got[key], ref[key]), key
    assert np.array_equal(np.nan_to_num(got["dev"], nan=-1), np.nan_to_num(ref["dev"], nan=-1))


def test_missing_query_row_is_an_index_error(validating):
    """Same row count, but the first query row replaced by a candidate."""
    need_gpu()
    case, cfg, layer, rope, ws = _setup()
    T, n_ctx, L0 = P.T, P.n_ctx, case["L0"]
    cand = np.arange(L0, n_ctx)
    s_in = np.concatenate([cand[:11], np.arange(n_ctx + 1, T)])             # 11 + (q - 1) rows, n_ctx missing
    st, out = _call(cfg, layer, rope, ws, case, s_in, None, 5)
    assert st == 3 and np.all(out["s_out"] == -5)


def test_select_validation(validating):
    need_gpu()
    cfg = F.config_of(P)
    n, k, T = 64, 10, P.T
    ws = F.workspace(cfg, T, n)
    sel = torch.full((k,), -5, dtype=torch.int32, device="cuda")
    d = torch.rand(n, device="cuda")
    d[17] = float("nan")
    with pytest.raises(F.CacheBlendError) as e:
        F.select_hkvd(cfg, None, None, T, None, n, k, d, sel, ws)
    assert e.value.status == 1 and torch.all(sel == -5)
    kn = torch.zeros((n, P.kv_dim), dtype=torch.bfloat16, device="cuda")
    kr = torch.zeros((T, P.kv_dim), dtype=torch.bfloat16, device="cuda")
    rows = torch.arange(n, dtype=torch.int32, device="cuda")
    rows[3] = T
    with pytest.raises(F.CacheBlendError) as e:
        F.select_hkvd(cfg, kn, kr, T, rows, n, k, torch.zeros(n, device="cuda"), sel, ws)
    assert e.value.status == 3 and torch.all(sel == -5)
    rows[3] = 3
    F.select_hkvd(cfg, kn, kr, T, rows, n, k, torch.zeros(n, device="cuda"), sel, ws)
    torch.cuda.synchronize()
    assert sel.cpu().numpy().tolist() == list(range(k))       # all deviations 0: the first k rows


def test_batch_validation(validating):
    """Two requests; the second one's rows run past its own cache."""
    need_gpu()
    case, cfg, layer, rope, ws = _setup()
    T, n_ctx, L0 = P.T, P.n_ctx, case["L0"]
    reqs, rows = [], []
    for j in range(2):
        reqs.append(dict(k_cache=dev(case["k"], torch.bfloat16), v_cache=dev(case["v"], torch.bfloat16), T=T,
                         n_ctx=n_ctx, first_chunk_len=L0, m_in=T - L0, k_out=20))
        rows.append(np.arange(L0, T))
    bad = [r.copy() for r in rows]
    bad[1][4] = bad[1][3]                                                   # a repeated row
    m_tot = 2 * (T - L0)
    ws2 = F.workspace(cfg, T, m_tot)
    for s_list, want in ((bad, 3), (rows, 0)):
        s_t = dev(np.concatenate(s_list).astype(np.int32), torch.int32)
        hid = dev(np.concatenate([case["hidden"][r] for r in rows]), torch.bfloat16)
        hout = torch.full((m_tot, P.d_model), 7.0, dtype=torch.bfloat16, device="cuda")
        dv = torch.full((m_tot,), 7.0, dtype=torch.float32, device="cuda")
        so = torch.full((m_tot,), -5, dtype=torch.int32, device="cuda")
        try:
            F.blend_batch(cfg, layer, rope, reqs, s_t, hid, hout, dv, so, ws2)
            st = 0
        except F.CacheBlendError as e:
            st = e.status
        torch.cuda.synchronize()
        assert st == want
        if want:
            assert torch.all(so == -5) and torch.all(dv == 7.0)
        else:
            assert torch.all(so[:2 * (20 + T - n_ctx)] >= L0)
