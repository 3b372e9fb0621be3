"""Host-side parts of bench.py's contract, on the CPU: more than one GPU is
refused before anything touches a device, the committed HBM-traffic entry is
reported only while the kernel sources it was measured on are unchanged, and
the layer's FLOP count matches the workload's closed form."""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_entry_follows_the_sources(tmp_path, monkeypatch):
    b = _bench()
    assert b.measured_traffic("gemm_gateup") is not None, "the committed entry matches the committed sources"
    assert b.measured_traffic("gemm_down") is None, "an entry names one kernel"
    # a changed source: the entry no longer applies
    src = tmp_path / "gemm.hip"
    src.write_bytes(open(os.path.join(ROOT, b.TRAFFIC_SOURCES[0]), "rb").read() + b"\n// changed\n")
    monkeypatch.setattr(b, "TRAFFIC_SOURCES", (str(src), b.TRAFFIC_SOURCES[1]))
    monkeypatch.setattr(b, "ROOT", ROOT)   # absolute paths join to themselves
    assert b.measured_traffic("gemm_gateup") is None


def test_layer_flops_closed_form():
    b = _bench()
    from rag_kv_cache_layer_amd import synth
    p = synth.PRESETS["llama8b_layer"]
    m = 493
    positions = np.arange(m)
    g = b.layer_flops(p, m, m, positions)
    d, F = p.d_model, p.ffn_dim
    qkv = p.q_dim + 2 * p.kv_dim
    assert g["gemm_qkv"] == 2 * m * d * qkv
    assert g["gemm_gateup"] == 2 * m * d * 2 * F
    assert g["gemm_down"] == 2 * m * F * d
    assert g["gemm_o"] == 2 * m * p.q_dim * d
    # attention: QK^T and PV over each row's keys 0..p (two multiply-adds per key and dim, every head)
    assert g["attention"] == 4 * p.head_dim * p.n_q_heads * int(np.sum(positions + 1))
    # the projections of the 8B layer at 493 rows: 2 m P_layer = 215.0 GFLOP
    assert sum(g[k] for k in ("gemm_qkv", "gemm_o", "gemm_gateup", "gemm_down")) == pytest.approx(215.0e9, rel=2e-3)
