"""Python binding of libcacheblend.so (the CacheBlend fusor for gfx950).

Argument marshalling only: every step of the fusor runs in the library's HIP
kernels.  torch is used for device memory and streams.  The function names
and argument orders are those of ``include/cacheblend.h``; tensors are passed
as device pointers after a shape / dtype / device check.

The library must have been built (``python -m rag_kv_cache_layer_amd.build``
or ``__graft_entry__.build()``); importing this module never compiles, and a
missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
# CB_LIB selects another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("CB_LIB") or os.path.join(PKG, "libcacheblend.so")

CB_F32, CB_BF16 = 0, 1
_STATUS = {0: "CB_OK", 1: "CB_ERR_ARG", 2: "CB_ERR_SHAPE", 3: "CB_ERR_INDEX", 4: "CB_ERR_WORKSPACE",
           5: "CB_ERR_UNSUPPORTED", 6: "CB_ERR_HIP"}


class CacheBlendError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{where}: {_STATUS.get(status, status)}"
        if status == 6:
            msg += f" (hipError {hip_error})"
        super().__init__(msg)


class LayerConfig(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn_dim", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "w_q", "w_k", "w_v", "w_o", "mlp_norm", "w_gate", "w_up", "w_down",
                 "w_gateup_packed", "w_qkv_folded")]


class LayerWeightsFp8(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "w_qkv", "e_qkv", "w_o", "e_o", "mlp_norm", "w_gu", "e_gu", "w_down", "e_down")]


class RopeDev(ctypes.Structure):
    _fields_ = [("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p), ("n_pos", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rope_theta", ctypes.c_float)]


def rope_dev(cfg: "LayerConfig", cos_ptr: int, sin_ptr: int, n_pos: int) -> RopeDev:
    """cb_rope_dev for a table built for cfg (its head_dim and rope_theta)."""
    return RopeDev(cos_ptr, sin_ptr, n_pos, cfg.head_dim, cfg.rope_theta)


class BlendRequest(ctypes.Structure):
    _fields_ = [("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("T", ctypes.c_int32),
                ("n_ctx", ctypes.c_int32), ("first_chunk_len", ctypes.c_int32), ("m_in", ctypes.c_int32),
                ("k_out", ctypes.c_int32)]


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double),
                ("min_ms", ctypes.c_double), ("max_ms", ctypes.c_double)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F32P, I32P = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, \
        ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)
    CFG, W, R = ctypes.POINTER(LayerConfig), ctypes.POINTER(LayerWeights), ctypes.POINTER(RopeDev)
    sig = {
        "cb_rope_table": (I32, [CFG, I32, I32, F32P, F32P]),
        "cb_num_selected": (I32, [I32, I32, I32]),
        "cb_filter_schedule": (I32, [I32, I32, I32, I32, I32, I32P]),
        "cb_workspace_size": (SZ, [CFG, I32, I32]),
        "cb_status_string": (ctypes.c_char_p, [I32]),
        "cb_last_hip_error": (I32, []),
        "cb_set_validate": (I32, [I32]),
        "cb_profile_begin": (I32, []),
        "cb_profile_end": (I32, [ctypes.POINTER(KernelStat), I32]),
        "cb_rope_shift": (I32, [CFG, R, P, I64, I32, I32, I32P, I32, P]),
        "cb_select_hkvd": (I32, [CFG, P, P, I32, P, I32, I32, P, P, P, SZ, P]),
        "cb_blend_layer": (I32, [CFG, W, R, P, P, I32, I32, I32, P, I32, P, P, I32, P, P, P, I32P, P, SZ, P]),
        "cb_blend_layer_realign": (I32, [CFG, W, R, P, P, I32, I32P, I32, P, I32, P, P, I32, P, P, P, I32P, P, SZ,
                                         P]),
        "cb_full_prefill_layer": (I32, [CFG, W, R, P, I32, I32, P, P, P, P, SZ, P]),
        "cb_blend_batch": (I32, [CFG, W, R, I32, ctypes.POINTER(BlendRequest), P, P, P, P, P, I32P, P, SZ, P]),
        "cb_stack_workspace_size": (SZ, [CFG, I32]),
        "cb_quantize_fp8": (I32, [I32, P, I32, I32, P, P, P]),
        "cb_gemm_fp8_workspace_size": (SZ, [I32, I32, I32]),
        "cb_gemm_fp8": (I32, [I32, I32, I32, P, P, P, P, P, I32, I32, P, SZ, P]),
        "cb_gemm_fp8_noalloc": (I32, [I32, I32, I32, P, P, P, P, P, I32, I32, P]),
        "cb_stream_copy": (I32, [P, P, SZ, P]),
        "cb_workspace_q_offset": (SZ, [CFG, I32]),
        "cb_analytics_workspace_size": (SZ, [I32, I32, I32]),
        "cb_attention_deviation": (I32, [CFG, I32, P, P, P, P, I32, P, P, P, SZ, P]),
        "cb_spearman": (I32, [P, P, I32, P, P, SZ, P]),
        "cb_top_share": (I32, [P, I32, I32, P, P, SZ, P]),
        "cb_pick_ratio": (I32, [ctypes.c_double, ctypes.c_double, I32, ctypes.c_double, I32]),
        "cb_blend_stack": (I32, [CFG, I32, W, R, P, P, I64, P, P, I32, I32P, I32, I32, P, I32P, P, P, P, I32P, P, SZ,
                                 P, P]),
        "cb_blend_stack_kv8": (I32, [CFG, I32, W, R, P, P, I64, P, P, P, P, I32, I32P, I32, I32, P, I32P, P, P, P,
                                     I32P, P, SZ, P, P]),
        "cb_kv_from_fp8": (I32, [CFG, R, P, P, P, P, I32, I32, I32, P, P, I64, I32, I32P, I32, I32, P]),
        "cb_workspace_size_fp8": (SZ, [CFG, I32, I32]),
        "cb_pack_gateup_size": (SZ, [CFG]),
        "cb_pack_gateup": (I32, [CFG, P, P, P, P]),
        "cb_fold_qkv_size": (SZ, [CFG]),
        "cb_fold_qkv": (I32, [CFG, W, P, P]),
        "cb_blend_layer_fp8": (I32, [CFG, ctypes.POINTER(LayerWeightsFp8), R, P, P, I32, I32, I32, P, I32, P, P, I32,
                                     P, P, P, I32P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def set_validate(on: bool) -> bool:
    """cb_set_validate for this thread; returns the previous setting."""
    return bool(lib().cb_set_validate(1 if on else 0))


def _check(status: int, where: str):
    if status != 0:
        raise CacheBlendError(status, where, lib().cb_last_hip_error())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def make_config(d_model: int, n_q_heads: int, n_kv_heads: int, head_dim: int, ffn_dim: int,
                rope_theta: float, rms_eps: float, dtype: str) -> LayerConfig:
    return LayerConfig(int(d_model), int(n_q_heads), int(n_kv_heads), int(head_dim), int(ffn_dim),
                       float(rope_theta), float(rms_eps), CB_BF16 if dtype == "bf16" else CB_F32)


def config_of(p) -> LayerConfig:
    """LayerConfig from an object with the preset fields (d_model, n_q_heads, ...)."""
    return make_config(p.d_model, p.n_q_heads, p.n_kv_heads, p.head_dim, p.ffn_dim, p.rope_theta, p.rms_eps,
                       p.dtype)


def _torch():
    import torch
    return torch


def torch_dtype(cfg: LayerConfig):
    torch = _torch()
    return torch.bfloat16 if cfg.dtype == CB_BF16 else torch.float32


def _dptr(t, name: str, dtype=None, numel: Optional[int] = None):
    """Device pointer of a contiguous CUDA/HIP tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------------------
# host helpers (no device needed)
# ---------------------------------------------------------------------------

def rope_table(cfg: LayerConfig, pos_begin: int, n_pos: int):
    """(cos, sin) fp32 [n_pos][hd/2] from cb_rope_table."""
    half = cfg.head_dim // 2
    cos = np.empty((n_pos, half), dtype=np.float32)
    sin = np.empty((n_pos, half), dtype=np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    _check(lib().cb_rope_table(ctypes.byref(cfg), pos_begin, n_pos, cos.ctypes.data_as(fp), sin.ctypes.data_as(fp)),
           "cb_rope_table")
    return cos, sin


def num_selected(r_e4: int, n_ctx: int, n_cand: int) -> int:
    return int(lib().cb_num_selected(r_e4, n_ctx, n_cand))


def filter_schedule(n_layers: int, r_first_e4: int, r_last_e4: int, n_ctx: int, n_cand: int):
    out = (ctypes.c_int32 * n_layers)()
    _check(lib().cb_filter_schedule(n_layers, r_first_e4, r_last_e4, n_ctx, n_cand, out), "cb_filter_schedule")
    return [int(x) for x in out]


def workspace_size(cfg: LayerConfig, T: int, m_max: int) -> int:
    return int(lib().cb_workspace_size(ctypes.byref(cfg), T, m_max))


def stack_workspace_size(cfg: LayerConfig, T: int) -> int:
    return int(lib().cb_stack_workspace_size(ctypes.byref(cfg), T))


def pick_ratio(t_prefill_us: float, kv_bytes_per_token: float, n_tokens: int, link_bytes_per_us: float,
               r_min_e4: int = 1500) -> int:
    """Loading controller's recompute ratio in units of 1e-4 (cb_pick_ratio)."""
    r = int(lib().cb_pick_ratio(float(t_prefill_us), float(kv_bytes_per_token), int(n_tokens),
                                float(link_bytes_per_us), int(r_min_e4)))
    if r < 0:
        raise CacheBlendError(1, "cb_pick_ratio")
    return r


def status_string(s: int) -> str:
    return lib().cb_status_string(s).decode()


def profile_begin():
    _check(lib().cb_profile_begin(), "cb_profile_begin")


def profile_end() -> Dict[str, dict]:
    out = (KernelStat * 64)()
    n = lib().cb_profile_end(out, 64)
    if n < 0:
        raise CacheBlendError(6, "cb_profile_end", lib().cb_last_hip_error())
    return {out[i].name.decode(): {"launches": out[i].launches, "total_ms": out[i].total_ms,
                                   "min_ms": out[i].min_ms, "max_ms": out[i].max_ms} for i in range(min(n, 64))}


# ---------------------------------------------------------------------------
# device objects
# ---------------------------------------------------------------------------

class DeviceRope:
    """RoPE table (cb_rope_table) for positions 0 .. n_pos-1, resident on the device."""

    def __init__(self, cfg: LayerConfig, n_pos: int, device="cuda"):
        torch = _torch()
        c, s = rope_table(cfg, 0, n_pos)
        self.cos = torch.from_numpy(c).to(device)
        self.sin = torch.from_numpy(s).to(device)
        self.struct = rope_dev(cfg, self.cos.data_ptr(), self.sin.data_ptr(), n_pos)


class DeviceLayer:
    """One layer's weights on the device (nn.Linear layout, cfg dtype; gains fp32)."""

    NAMES = ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down")

    def __init__(self, cfg: LayerConfig, weights: Dict[str, object], device="cuda"):
        torch = _torch()
        dt = torch_dtype(cfg)
        self.t = {}
        for k in self.NAMES:
            v = weights[k]
            v = v if isinstance(v, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(v))
            self.t[k] = v.to(device=device, dtype=dt).contiguous()
        for k in ("attn_norm", "mlp_norm"):
            v = weights[k]
            v = v if isinstance(v, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(v))
            self.t[k] = v.to(device=device, dtype=torch.float32).contiguous()
        self.struct = LayerWeights(*[self.t[n].data_ptr() for n in
                                     ("attn_norm", "w_q", "w_k", "w_v", "w_o", "mlp_norm", "w_gate", "w_up",
                                      "w_down")])
        self.cfg = cfg

    def pack_gateup(self, stream=None) -> "DeviceLayer":
        """cb_pack_gateup: repack W_gate and W_up once into the gate/up
        kernel's streaming order; the layer's calls then read the packed copy
        (same results, bit for bit).  Returns self."""
        torch = _torch()
        n = int(lib().cb_pack_gateup_size(ctypes.byref(self.cfg)))
        if n == 0:
            raise CacheBlendError(5, "cb_pack_gateup_size")
        self.t["w_gateup_packed"] = torch.empty(n, dtype=torch.uint8, device=self.t["w_gate"].device)
        _check(lib().cb_pack_gateup(ctypes.byref(self.cfg), _dptr(self.t["w_gate"], "w_gate"),
                                    _dptr(self.t["w_up"], "w_up"), _dptr(self.t["w_gateup_packed"], "packed"),
                                    _stream(stream)), "cb_pack_gateup")
        self.struct.w_gateup_packed = self.t["w_gateup_packed"].data_ptr()
        return self

    def fold_qkv(self, stream=None) -> "DeviceLayer":
        """cb_fold_qkv: [W_q; W_k; W_v] with the attention RMSNorm gain folded
        in, once; the layer's bf16 calls then run the RMSNorm inside the QKV
        projection.  Returns self."""
        torch = _torch()
        n = int(lib().cb_fold_qkv_size(ctypes.byref(self.cfg)))
        if n == 0:
            raise CacheBlendError(5, "cb_fold_qkv_size")
        self.t["w_qkv_folded"] = torch.empty(n, dtype=torch.uint8, device=self.t["w_q"].device)
        _check(lib().cb_fold_qkv(ctypes.byref(self.cfg), ctypes.byref(self.struct),
                                 _dptr(self.t["w_qkv_folded"], "out"), _stream(stream)), "cb_fold_qkv")
        self.struct.w_qkv_folded = self.t["w_qkv_folded"].data_ptr()
        return self


class DeviceLayerFp8:
    """One layer's weights as 8-bit E4M3 codes + per-row exponents on the
    device (cb_layer_weights_fp8): weights maps "w_qkv", "w_o", "w_gu",
    "w_down" to (codes uint8 [rows][in], exps int32 [rows]) -- QKV rows are
    W_q, W_k, W_v stacked, gate/up rows W_gate then W_up -- and "attn_norm",
    "mlp_norm" to fp32 gains."""

    NAMES = ("w_qkv", "w_o", "w_gu", "w_down")

    def __init__(self, cfg: LayerConfig, weights: Dict[str, object], device="cuda"):
        torch = _torch()
        conv = lambda v: v if isinstance(v, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(v))
        self.t = {}
        for k in self.NAMES:
            c, e = weights[k]
            self.t[k] = conv(c).to(device=device, dtype=torch.uint8).contiguous()
            self.t["e" + k[1:]] = conv(e).to(device=device, dtype=torch.int32).contiguous()
        for k in ("attn_norm", "mlp_norm"):
            self.t[k] = conv(weights[k]).to(device=device, dtype=torch.float32).contiguous()
        self.struct = LayerWeightsFp8(*[self.t[n].data_ptr() for n in
                                        ("attn_norm", "w_qkv", "e_qkv", "w_o", "e_o", "mlp_norm", "w_gu", "e_gu",
                                         "w_down", "e_down")])

    @classmethod
    def quantized(cls, cfg: LayerConfig, layer: "DeviceLayer", device="cuda") -> "DeviceLayerFp8":
        """Quantize a DeviceLayer's weights on the device (cb_quantize_fp8)."""
        torch = _torch()
        t = layer.t
        w = {"w_qkv": quantize_fp8(torch.cat([t["w_q"], t["w_k"], t["w_v"]])),
             "w_o": quantize_fp8(t["w_o"]), "w_gu": quantize_fp8(torch.cat([t["w_gate"], t["w_up"]])),
             "w_down": quantize_fp8(t["w_down"]), "attn_norm": t["attn_norm"], "mlp_norm": t["mlp_norm"]}
        return cls(cfg, w, device)


def workspace_fp8(cfg: LayerConfig, T: int, m_max: int, device="cuda"):
    torch = _torch()
    n = int(lib().cb_workspace_size_fp8(ctypes.byref(cfg), T, m_max))
    if n == 0:
        raise CacheBlendError(1, "cb_workspace_size_fp8")
    return torch.empty(n, dtype=torch.uint8, device=device)


def workspace(cfg: LayerConfig, T: int, m_max: int, device="cuda"):
    torch = _torch()
    n = workspace_size(cfg, T, m_max)
    if n == 0:
        raise CacheBlendError(1, "cb_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# device calls
# ---------------------------------------------------------------------------

def rope_shift(cfg: LayerConfig, rope: DeviceRope, k_cache, layer_stride: int, n_layers: int, T: int,
               chunk_offsets: Sequence[int], stream=None):
    offs = np.ascontiguousarray(np.asarray(chunk_offsets, dtype=np.int32))
    kv = cfg.n_kv_heads * cfg.head_dim
    need = (n_layers - 1) * layer_stride + T * kv if n_layers > 0 else 0
    _check(lib().cb_rope_shift(ctypes.byref(cfg), ctypes.byref(rope.struct),
                               _dptr(k_cache, "k_cache", torch_dtype(cfg), need), layer_stride, n_layers, T,
                               offs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(offs) - 1,
                               _stream(stream)), "cb_rope_shift")


def workspace_q(cfg: LayerConfig, ws, T: int, rows: int):
    """View of the Q rows [rows][n_q][hd] that the last cb_blend_layer (with
    this T) or cb_full_prefill_layer (over T rows) left in workspace ws
    (cb_workspace_q_offset); valid until the next call on ws."""
    torch = _torch()
    off = int(lib().cb_workspace_q_offset(ctypes.byref(cfg), T))
    if off == 0:
        raise CacheBlendError(1, "cb_workspace_q_offset")
    dt = torch_dtype(cfg)
    es = torch.empty((), dtype=dt).element_size()
    n = rows * cfg.n_q_heads * cfg.head_dim * es
    return ws[off:off + n].view(dt).view(rows, cfg.n_q_heads, cfg.head_dim)


def _analytics_ws(m: int, n_q: int, n: int, device):
    torch = _torch()
    return torch.empty(int(lib().cb_analytics_workspace_size(m, n_q, n)), dtype=torch.uint8, device=device)


def attention_deviation(cfg: LayerConfig, q_a, k_a, q_b, k_b, last_key, stream=None):
    """cb_attention_deviation: (||A_a - A_b||_F^2, ||A_b||_F^2) as Python floats."""
    torch = _torch()
    dt = torch_dtype(cfg)
    m = q_a.shape[0]
    T = k_a.shape[0]
    kv = cfg.n_kv_heads * cfg.head_dim
    qd = cfg.n_q_heads * cfg.head_dim
    out = torch.empty(2, dtype=torch.float64, device=q_a.device)
    ws = _analytics_ws(m, cfg.n_q_heads, 0, q_a.device)
    _check(lib().cb_attention_deviation(ctypes.byref(cfg), m, _dptr(q_a, "q_a", dt, m * qd),
                                        _dptr(k_a, "k_a", dt, T * kv), _dptr(q_b, "q_b", dt, m * qd),
                                        _dptr(k_b, "k_b", dt, T * kv), T, _dptr(last_key, "last_key", torch.int32, m),
                                        _dptr(out, "out"), _dptr(ws, "ws"), ws.numel(), _stream(stream)),
           "cb_attention_deviation")
    o = out.cpu()
    return float(o[0]), float(o[1])


def spearman(x, y, stream=None) -> float:
    """cb_spearman of two device fp32 vectors."""
    torch = _torch()
    n = x.numel()
    out = torch.empty(1, dtype=torch.float64, device=x.device)
    ws = _analytics_ws(0, 0, n, x.device)
    _check(lib().cb_spearman(_dptr(x, "x", torch.float32, n), _dptr(y, "y", torch.float32, n), n, _dptr(out, "out"),
                             _dptr(ws, "ws"), ws.numel(), _stream(stream)), "cb_spearman")
    return float(out.cpu()[0])


def top_share(x, k: int, stream=None) -> float:
    """cb_top_share: share of sum(x) held by its k largest values."""
    torch = _torch()
    n = x.numel()
    out = torch.empty(1, dtype=torch.float64, device=x.device)
    ws = _analytics_ws(0, 0, n, x.device)
    _check(lib().cb_top_share(_dptr(x, "x", torch.float32, n), n, k, _dptr(out, "out"), _dptr(ws, "ws"), ws.numel(),
                              _stream(stream)), "cb_top_share")
    return float(out.cpu()[0])


def stream_copy(src, dst, stream=None):
    """cb_stream_copy: dst <- src (same byte size), the HBM reference copy."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("stream_copy: sizes differ")
    _check(lib().cb_stream_copy(_dptr(src, "src"), _dptr(dst, "dst"), n, _stream(stream)), "cb_stream_copy")


def select_hkvd(cfg: LayerConfig, k_new, k_ref, T: int, cand_rows, n: int, k: int, dev, sel_out, ws, stream=None):
    torch = _torch()
    kv = cfg.n_kv_heads * cfg.head_dim
    _check(lib().cb_select_hkvd(ctypes.byref(cfg), _dptr(k_new, "k_new", torch_dtype(cfg), n * kv),
                                _dptr(k_ref, "k_ref", torch_dtype(cfg), T * kv if k_new is not None else None),
                                T, _dptr(cand_rows, "cand_rows", torch.int32, n), n, k,
                                _dptr(dev, "dev", torch.float32, n), _dptr(sel_out, "sel_out", torch.int32, k),
                                _dptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)), "cb_select_hkvd")


def blend_layer(cfg: LayerConfig, layer: DeviceLayer, rope: DeviceRope, k_cache, v_cache, T: int, n_ctx: int,
                first_chunk_len: int, s_in, m_in: int, hidden_in, in_rows, k_out: int, hidden_out, dev_out, s_out,
                ws, stream=None) -> int:
    """One selective-recompute layer; returns m_out (rows of hidden_out / s_out written)."""
    torch = _torch()
    dt = torch_dtype(cfg)
    kv, d = cfg.n_kv_heads * cfg.head_dim, cfg.d_model
    m_exp = max(expected_m_out(T, n_ctx, m_in, k_out), 0)
    m_out = ctypes.c_int32(0)
    _check(lib().cb_blend_layer(ctypes.byref(cfg), ctypes.byref(layer.struct), ctypes.byref(rope.struct),
                                _dptr(k_cache, "k_cache", dt, T * kv), _dptr(v_cache, "v_cache", dt, T * kv), T,
                                n_ctx, first_chunk_len, _dptr(s_in, "s_in", torch.int32, m_in), m_in,
                                _dptr(hidden_in, "hidden_in", dt, (T if in_rows is not None else m_in) * d),
                                _dptr(in_rows, "in_rows", torch.int32, m_in), k_out,
                                _dptr(hidden_out, "hidden_out", dt, m_exp * d),
                                _dptr(dev_out, "dev_out", torch.float32, m_in),
                                _dptr(s_out, "s_out", torch.int32, m_exp), ctypes.byref(m_out),
                                _dptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)), "cb_blend_layer")
    return int(m_out.value)


def blend_layer_realign(cfg: LayerConfig, layer: DeviceLayer, rope: DeviceRope, k_cache, v_cache, T: int,
                        chunk_offsets: Sequence[int], s_in, m_in: int, hidden_in, in_rows, k_out: int, hidden_out,
                        dev_out, s_out, ws, stream=None) -> int:
    """cb_blend_layer_realign: the layer's RoPE re-alignment and one selective-
    recompute layer in one call (k_cache still at chunk-local positions);
    returns m_out."""
    torch = _torch()
    dt = torch_dtype(cfg)
    kv, d = cfg.n_kv_heads * cfg.head_dim, cfg.d_model
    offs = np.ascontiguousarray(np.asarray(chunk_offsets, dtype=np.int32))
    n_ctx = int(offs[-1]) if len(offs) else 0
    m_exp = max(expected_m_out(T, n_ctx, m_in, k_out), 0)
    m_out = ctypes.c_int32(0)
    _check(lib().cb_blend_layer_realign(ctypes.byref(cfg), ctypes.byref(layer.struct), ctypes.byref(rope.struct),
                                        _dptr(k_cache, "k_cache", dt, T * kv), _dptr(v_cache, "v_cache", dt, T * kv),
                                        T, offs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(offs) - 1,
                                        _dptr(s_in, "s_in", torch.int32, m_in), m_in,
                                        _dptr(hidden_in, "hidden_in", dt, (T if in_rows is not None else m_in) * d),
                                        _dptr(in_rows, "in_rows", torch.int32, m_in), k_out,
                                        _dptr(hidden_out, "hidden_out", dt, m_exp * d),
                                        _dptr(dev_out, "dev_out", torch.float32, m_in),
                                        _dptr(s_out, "s_out", torch.int32, m_exp), ctypes.byref(m_out),
                                        _dptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)),
           "cb_blend_layer_realign")
    return int(m_out.value)


def blend_layer_fp8(cfg: LayerConfig, layer: DeviceLayerFp8, rope: DeviceRope, k_cache, v_cache, T: int, n_ctx: int,
                    first_chunk_len: int, s_in, m_in: int, hidden_in, in_rows, k_out: int, hidden_out, dev_out,
                    s_out, ws, stream=None) -> int:
    """cb_blend_layer_fp8: blend_layer with 8-bit projections; returns m_out."""
    torch = _torch()
    dt = torch_dtype(cfg)
    kv, d = cfg.n_kv_heads * cfg.head_dim, cfg.d_model
    m_exp = max(expected_m_out(T, n_ctx, m_in, k_out), 0)
    m_out = ctypes.c_int32(0)
    _check(lib().cb_blend_layer_fp8(ctypes.byref(cfg), ctypes.byref(layer.struct), ctypes.byref(rope.struct),
                                    _dptr(k_cache, "k_cache", dt, T * kv), _dptr(v_cache, "v_cache", dt, T * kv), T,
                                    n_ctx, first_chunk_len, _dptr(s_in, "s_in", torch.int32, m_in), m_in,
                                    _dptr(hidden_in, "hidden_in", dt, (T if in_rows is not None else m_in) * d),
                                    _dptr(in_rows, "in_rows", torch.int32, m_in), k_out,
                                    _dptr(hidden_out, "hidden_out", dt, m_exp * d),
                                    _dptr(dev_out, "dev_out", torch.float32, m_in),
                                    _dptr(s_out, "s_out", torch.int32, m_exp), ctypes.byref(m_out),
                                    _dptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)),
           "cb_blend_layer_fp8")
    return int(m_out.value)


def blend_batch(cfg: LayerConfig, layer: DeviceLayer, rope: DeviceRope, reqs: Sequence[dict], s_in, hidden_in,
                hidden_out, dev_out, s_out, ws, stream=None):
    """One fusor layer for several requests (cb_blend_batch).  reqs: dicts with
    k_cache, v_cache (device tensors), T, n_ctx, first_chunk_len, m_in, k_out.
    s_in / hidden_in / dev_out hold the requests' rows one after another;
    hidden_out / s_out receive the kept rows likewise.  Returns m_out per
    request."""
    torch = _torch()
    dt = torch_dtype(cfg)
    kv, d = cfg.n_kv_heads * cfg.head_dim, cfg.d_model
    n = len(reqs)
    arr = (BlendRequest * n)()
    m_in_tot = m_out_tot = 0
    for i, r in enumerate(reqs):
        arr[i] = BlendRequest(_dptr(r["k_cache"], "k_cache", dt, r["T"] * kv).value,
                              _dptr(r["v_cache"], "v_cache", dt, r["T"] * kv).value, r["T"], r["n_ctx"],
                              r["first_chunk_len"], r["m_in"], r["k_out"])
        m_in_tot += r["m_in"]
        m_out_tot += max(expected_m_out(r["T"], r["n_ctx"], r["m_in"], r["k_out"]), 0)
    m_out = (ctypes.c_int32 * n)()
    _check(lib().cb_blend_batch(ctypes.byref(cfg), ctypes.byref(layer.struct), ctypes.byref(rope.struct), n, arr,
                                _dptr(s_in, "s_in", torch.int32, m_in_tot),
                                _dptr(hidden_in, "hidden_in", dt, m_in_tot * d),
                                _dptr(hidden_out, "hidden_out", dt, m_out_tot * d),
                                _dptr(dev_out, "dev_out", torch.float32, m_in_tot),
                                _dptr(s_out, "s_out", torch.int32, m_out_tot), m_out,
                                _dptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)), "cb_blend_batch")
    return [int(x) for x in m_out]


def expected_m_out(T: int, n_ctx: int, m_in: int, k_out: int) -> int:
    """m_out of cb_blend_layer, known on the host before the call."""
    n_query = T - n_ctx
    return min(k_out, m_in - n_query) + n_query


def full_prefill_layer(cfg: LayerConfig, layer: DeviceLayer, rope: DeviceRope, hidden_in, T: int, pos0: int,
                       k_out, v_out, hidden_out, ws, stream=None):
    dt = torch_dtype(cfg)
    kv, d = cfg.n_kv_heads * cfg.head_dim, cfg.d_model
    _check(lib().cb_full_prefill_layer(ctypes.byref(cfg), ctypes.byref(layer.struct), ctypes.byref(rope.struct),
                                       _dptr(hidden_in, "hidden_in", dt, T * d), T, pos0,
                                       _dptr(k_out, "k_out", dt, T * kv), _dptr(v_out, "v_out", dt, T * kv),
                                       _dptr(hidden_out, "hidden_out", dt, T * d), _dptr(ws, "ws", _torch().uint8),
                                       ws.numel(), _stream(stream)), "cb_full_prefill_layer")


# ---------------------------------------------------------------------------
# stack driver (gradual filtering across layers)
# ---------------------------------------------------------------------------

def blend_stack(cfg: LayerConfig, layers: Sequence[DeviceLayer], rope: DeviceRope, k_caches, v_caches, T: int,
                chunk_offsets: Sequence[int], x_first, ks: Sequence[int], ws, stream=None, shift: bool = True):
    """Run the fusor through every layer (CacheBlend section 4.3, Figure 9).

    k_caches, v_caches: device [n_layers][T][n_kv][hd], each chunk's cached K/V
    in context order (keys at their local positions when shift=True, the
    re-alignment then runs once over all layers).  x_first: device [m0][d],
    the first layer's input for rows first_chunk_len .. T-1.  ks: per-layer
    k_out (filter_schedule).  Layer 0 recomputes every candidate; later layers
    recompute the rows the previous layer kept.  Every row count is known on
    the host, so nothing waits on the device.  Returns a list of per-layer
    dicts (s_in, dev, s_out, y) of device tensors; the last y holds the output
    of the rows the last layer kept."""
    torch = _torch()
    n_layers = len(layers)
    offs = [int(o) for o in chunk_offsets]
    n_ctx, L0 = offs[-1], offs[1] if len(offs) > 1 else offs[-1]
    kv = cfg.n_kv_heads * cfg.head_dim
    if shift:
        rope_shift(cfg, rope, k_caches, T * kv, n_layers, T, offs, stream)
    dev_ = x_first.device
    s = torch.arange(L0, T, dtype=torch.int32, device=dev_)
    x = x_first
    out = []
    for l in range(n_layers):
        m_in = s.numel()
        m_out = expected_m_out(T, n_ctx, m_in, ks[l])
        y = torch.empty((m_out, cfg.d_model), dtype=torch_dtype(cfg), device=dev_)
        s_out = torch.empty(m_out, dtype=torch.int32, device=dev_)
        dv = torch.empty(m_in, dtype=torch.float32, device=dev_)
        blend_layer(cfg, layers[l], rope, k_caches[l], v_caches[l], T, n_ctx, L0, s, m_in, x, None, ks[l], y, dv,
                    s_out, ws, stream)
        out.append({"s_in": s, "dev": dv, "s_out": s_out, "y": y})
        s, x = s_out, y
    return out


def stack_rows(T: int, chunk_offsets: Sequence[int], ks: Sequence[int]):
    """(m_in, m_out) per layer of cb_blend_stack, computed on the host."""
    offs = [int(o) for o in chunk_offsets]
    n_ctx = offs[-1]
    L0 = offs[1] if len(offs) > 2 else n_ctx
    q = T - n_ctx
    rows, m_in, m_out = T - L0, [], []
    for k in ks:
        m_in.append(rows)
        rows = min(int(k), rows - q) + q
        m_out.append(rows)
    return m_in, m_out


def blend_stack_native(cfg: LayerConfig, layers: Sequence[DeviceLayer], rope: DeviceRope, k_caches, v_caches,
                       T: int, chunk_offsets: Sequence[int], x_first, ks: Sequence[int], ws, k_src=None, v_src=None,
                       shift: bool = True, stream=None, copy_stream=None, k_src_exp=None, v_src_exp=None):
    """cb_blend_stack: the whole stack in one library call.

    k_caches, v_caches: device [n_layers][T][n_kv][hd].  k_src, v_src: None,
    or host tensors of the same shape (pinned for overlap) whose copies run on
    copy_stream (a torch stream; None = on `stream`).  With k_src_exp and
    v_src_exp (host int32 [n_layers][T][n_kv]) the sources are 8-bit E4M3
    codes (uint8) and cb_blend_stack_kv8 runs instead.  ws: uint8 device
    tensor of stack_workspace_size bytes.  Returns a list of per-layer dicts
    (dev, s_out as views into the concatenated outputs; y only for the last
    layer), like blend_stack."""
    torch = _torch()
    n = len(layers)
    dt = torch_dtype(cfg)
    kv, d = cfg.n_kv_heads * cfg.head_dim, cfg.d_model
    offs = np.ascontiguousarray(np.asarray(chunk_offsets, dtype=np.int32))
    ks_a = np.ascontiguousarray(np.asarray(ks, dtype=np.int32))
    if len(ks_a) != n:
        raise ValueError("one k_out per layer")
    m_in, m_out = stack_rows(T, offs, ks_a)
    dev_ = x_first.device
    s_all = torch.empty(max(sum(m_out), 1), dtype=torch.int32, device=dev_)
    dev_all = torch.empty(max(sum(m_in), 1), dtype=torch.float32, device=dev_)
    y = torch.empty((max(m_out[-1], 1), d), dtype=dt, device=dev_)
    W = (LayerWeights * n)(*[l.struct for l in layers])
    rows = (ctypes.c_int32 * (2 * n))()
    if (k_src is None) != (v_src is None) or (k_src_exp is None) != (v_src_exp is None):
        raise ValueError("k_src and v_src (and their exponents) go together")
    q8 = k_src_exp is not None
    if q8 and k_src is None:
        raise ValueError("exponents without 8-bit sources")
    src = []
    for name, t, want, numel in (("k_src", k_src, torch.uint8 if q8 else dt, n * T * kv),
                                 ("v_src", v_src, torch.uint8 if q8 else dt, n * T * kv),
                                 ("k_src_exp", k_src_exp, torch.int32, n * T * cfg.n_kv_heads),
                                 ("v_src_exp", v_src_exp, torch.int32, n * T * cfg.n_kv_heads)):
        if t is None:
            src.append(None)
            continue
        if t.is_cuda or not t.is_contiguous() or t.dtype != want or t.numel() < numel:
            raise ValueError(f"{name} must be a contiguous host tensor of {numel} {want} elements")
        src.append(ctypes.c_void_p(t.data_ptr()))
    cs = None if copy_stream is None else ctypes.c_void_p(copy_stream.cuda_stream)
    L0 = int(offs[1]) if len(offs) > 2 else int(offs[-1])
    common_head = (ctypes.byref(cfg), n, W, ctypes.byref(rope.struct), _dptr(k_caches, "k_caches", dt, n * T * kv),
                   _dptr(v_caches, "v_caches", dt, n * T * kv), T * kv)
    common_tail = (T, offs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(offs) - 1, 1 if shift else 0,
                   _dptr(x_first, "x_first", dt, (T - L0) * d), ks_a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                   _dptr(s_all, "s_out_all"), _dptr(dev_all, "dev_all"), _dptr(y, "hidden_out"), rows,
                   _dptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream), cs)
    if q8:
        _check(lib().cb_blend_stack_kv8(*common_head, src[0], src[2], src[1], src[3], *common_tail),
               "cb_blend_stack_kv8")
    else:
        _check(lib().cb_blend_stack(*common_head, src[0], src[1], *common_tail), "cb_blend_stack")
    out, oi, oo = [], 0, 0
    for l in range(n):
        out.append({"dev": dev_all[oi:oi + m_in[l]], "s_out": s_all[oo:oo + m_out[l]]})
        oi += m_in[l]
        oo += m_out[l]
    out[-1]["y"] = y[:m_out[-1]]
    return out


# ---------------------------------------------------------------------------
# fp8 E4M3 operands
# ---------------------------------------------------------------------------

def kv_from_fp8(cfg: LayerConfig, rope: Optional[DeviceRope], k_codes, k_exps, v_codes, v_exps, k_cache, v_cache,
                layer_stride: int, n_layers: int, T: int, chunk_offsets: Sequence[int], row_begin: int = 0,
                n_rows: Optional[int] = None, shift: bool = True, stream=None):
    """cb_kv_from_fp8: expand 8-bit K/V codes (device uint8 [n_layers][n_rows][n_kv][hd],
    exponents int32 [n_layers][n_rows][n_kv]) into rows row_begin.. of the caches."""
    torch = _torch()
    dt = torch_dtype(cfg)
    kv = cfg.n_kv_heads * cfg.head_dim
    n_rows = T - row_begin if n_rows is None else n_rows
    offs = np.ascontiguousarray(np.asarray(chunk_offsets, dtype=np.int32))
    need = (n_layers - 1) * layer_stride + T * kv if n_layers > 0 else 0
    nc, ne = n_layers * n_rows * kv, n_layers * n_rows * cfg.n_kv_heads
    _check(lib().cb_kv_from_fp8(ctypes.byref(cfg), ctypes.byref(rope.struct) if rope is not None else None,
                                _dptr(k_codes, "k_codes", torch.uint8, nc), _dptr(k_exps, "k_exps", torch.int32, ne),
                                _dptr(v_codes, "v_codes", torch.uint8, nc), _dptr(v_exps, "v_exps", torch.int32, ne),
                                n_layers, row_begin, n_rows, _dptr(k_cache, "k_cache", dt, need),
                                _dptr(v_cache, "v_cache", dt, need), layer_stride, T,
                                offs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(offs) - 1,
                                1 if shift else 0, _stream(stream)), "cb_kv_from_fp8")


def quantize_fp8(x, codes=None, exps=None, stream=None):
    """cb_quantize_fp8 of a device matrix x [rows][cols] (bf16 or fp32);
    returns (codes uint8 [rows][cols], exps int32 [rows])."""
    torch = _torch()
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if codes is None else codes
    exps = torch.empty(rows, dtype=torch.int32, device=x.device) if exps is None else exps
    src = CB_BF16 if x.dtype == torch.bfloat16 else CB_F32
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be bf16 or fp32")
    _check(lib().cb_quantize_fp8(src, _dptr(x, "x"), rows, cols, _dptr(codes, "codes", torch.uint8, rows * cols),
                                 _dptr(exps, "exps", torch.int32, rows), _stream(stream)), "cb_quantize_fp8")
    return codes, exps


def gemm_fp8(a, a_exp, b, b_exp, out, ws=None, stream=None):
    """cb_gemm_fp8: out [M][N] (bf16 or fp32) = (A B^T) scaled by the row
    exponents; a [M][K], b [N][K] uint8 codes."""
    torch = _torch()
    M, K = a.shape
    N = b.shape[0]
    need = int(lib().cb_gemm_fp8_workspace_size(M, N, K))
    if need and (ws is None or ws.numel() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=a.device)
    od = CB_BF16 if out.dtype == torch.bfloat16 else CB_F32
    _check(lib().cb_gemm_fp8(M, N, K, _dptr(a, "a", torch.uint8, M * K), _dptr(a_exp, "a_exp", torch.int32, M),
                             _dptr(b, "b", torch.uint8, N * K), _dptr(b_exp, "b_exp", torch.int32, N),
                             _dptr(out, "out", None, M * out.stride(0)), out.stride(0), od,
                             _dptr(ws, "ws") if need else None, ws.numel() if need else 0, _stream(stream)),
           "cb_gemm_fp8")
    return out


GEMM_FP8_SCRATCH_BYTES = 32 << 20   # CB_GEMM_FP8_SCRATCH_BYTES


def gemm_fp8_noalloc(a, a_exp, b, b_exp, out, stream=None):
    """cb_gemm_fp8_noalloc: gemm_fp8 with the split-K partials in the
    library's static per-GPU array (no workspace argument, no allocation)."""
    torch = _torch()
    M, K = a.shape
    N = b.shape[0]
    od = CB_BF16 if out.dtype == torch.bfloat16 else CB_F32
    _check(lib().cb_gemm_fp8_noalloc(M, N, K, _dptr(a, "a", torch.uint8, M * K),
                                     _dptr(a_exp, "a_exp", torch.int32, M), _dptr(b, "b", torch.uint8, N * K),
                                     _dptr(b_exp, "b_exp", torch.int32, N),
                                     _dptr(out, "out", None, M * out.stride(0)), out.stride(0), od,
                                     _stream(stream)), "cb_gemm_fp8_noalloc")
    return out
