"""Throughput of the CacheBlend fusor layer on one MI355X.

Workload: the Llama-3-8B-shaped bf16 layer (d_model 4096, 32 query / 8 KV
heads of 128, FFN 14336, RoPE base 500000) with 6 retrieved chunks of 512
tokens and a 32-token query (3104 tokens), recompute ratio r = 0.15 (461
HKVD tokens + 32 query rows).  Weights N(0, 0.02) and chunk / query
embeddings N(0, 1) are seeded synthetic values; the cached K/V of each chunk
come from an isolated prefill at position 0 and the hidden states from a full
prefill of the same layer (set-up, untimed, on the GPU).

One step is one fusor layer in one call (cb_blend_layer_realign): the RoPE
re-alignment of that layer's cached keys and the selective recompute of the
HKVD rows (gather + RMSNorm, QKV with RoPE, K deviation and K/V scatter,
top-k, partial causal GQA attention, O projection, SwiGLU MLP).  With
--separate-shift the step is cb_rope_shift followed by cb_blend_layer (the
same results, one launch more).
value = context tokens blended per second = T / step time.

Prints one JSON line.  --gpus above 1 is refused: the benchmark measures one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
CALIB_COPY_BYTES = 512 << 20   # reference copy for the counter calibration (twice the Infinity Cache)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--separate-shift", action="store_true",
                    help="time cb_rope_shift + cb_blend_layer instead of the one-call cb_blend_layer_realign")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--extra", action="store_true", help="also time the select call and full prefill")
    ap.add_argument("--batch", type=int, default=0,
                    help="also time one batched fusor layer (cb_blend_batch) over this many copies of the request")
    ap.add_argument("--pipeline", action="store_true",
                    help="also measure the 32-layer stack with its KV loaded from pinned host memory "
                         "(loading alone, recompute alone, both pipelined)")
    ap.add_argument("--fp8", action="store_true",
                    help="also time the layer's four projections with fp8 E4M3 operands (cb_quantize_fp8 + "
                         "cb_gemm_fp8) at the same row count")
    ap.add_argument("--analytics", action="store_true",
                    help="also run the deviation analytics (attention deviation vs r, deviation "
                         "concentration, neighbour-layer rank correlation) on the 32-layer stack")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the blend step and full prefill of the 8B layer over 4/16/32 chunks x 512 + 64 "
                         "tokens at r = 0.05, 0.10, 0.15, 0.30, 1.0")
    ap.add_argument("--llama70b", action="store_true",
                    help="also time the blend call of one Llama-70B-shaped layer (8 x 500 + 32 tokens, r=0.15)")
    ap.add_argument("--cpu-extra", action="store_true",
                    help="also time the CPU oracle on the other workloads: the tiny fp32 layer (1 thread and all), "
                         "full prefill of the 8B layer, the 4-chunk sweep layer at r = 0.15 and 1, and spot layers "
                         "of the 32-layer 8B and 80-layer 70B stacks (scaled by the layer count, an estimate)")
    ap.add_argument("--hbm-only", action="store_true",
                    help="only the cold, large launches of the bandwidth-bound kernels (stack-wide RoPE shift, "
                         "deviation over 15872 candidates, 8-bit KV expansion of the stack) and the streaming "
                         "copy they are compared with; one JSON line")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one untimed 512 MiB device-to-device copy first (a known-size reference "
                         "for the HBM byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gateup_llama8b_hbm_traffic.md")
TRAFFIC_SOURCES = ("rag_kv_cache_layer_amd/csrc/gemm.hip", "rag_kv_cache_layer_amd/csrc/cb_internal.h")


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when there is none or the kernel sources changed since
    the counters were taken (the summary stores their SHA-256)."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
        entry = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if entry.get("kernel") != kernel or entry.get("source_sha256") != h.hexdigest():
        return None
    return int(entry["traffic_bytes"])


def layer_flops(p, m_in, m_out, positions):
    d, q, kv, F = p.d_model, p.q_dim, p.kv_dim, p.ffn_dim
    g = {"gemm_qkv": 2 * m_in * d * (q + 2 * kv), "gemm_o": 2 * m_out * q * d,
         "gemm_gateup": 2 * m_out * d * 2 * F, "gemm_down": 2 * m_out * F * d}
    g["attention"] = int(4 * p.head_dim * p.n_q_heads * np.sum(np.asarray(positions, np.int64) + 1))
    return g


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the library runs on one GPU", file=sys.stderr)
        sys.exit(2)
    import torch
    from rag_kv_cache_layer_amd import fusor as F
    from rag_kv_cache_layer_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    F.lib()   # fails loudly when the library is missing
    if args.hbm_only:
        out = hbm_kernels_measure()
        print(json.dumps(out))
        return
    log("library loaded; generating inputs")
    p = synth.PRESETS["llama8b_layer"]
    seed = args.seed
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    cfg = F.config_of(p)
    T, n_ctx, d, kvd = p.T, p.n_ctx, p.d_model, p.kv_dim
    order = synth.chunk_order(p, seed)
    offs = synth.chunk_offsets(p, order)
    L0 = int(offs[1])
    n_cand = n_ctx - L0
    k = F.num_selected(p.r_e4, n_ctx, n_cand)

    # ---------------- set-up (untimed) ----------------
    w = synth.layer_weights(p, seed, 0)
    # W_gate / W_up repacked once into the gate/up kernel's streaming order
    # (a model-load step, untimed; results are bit-identical to row-major),
    # and the attention RMSNorm gain folded into W_q/W_k/W_v once so that the
    # RMSNorm runs inside the QKV projection
    layer = F.DeviceLayer(cfg, w, dev).pack_gateup().fold_qkv()
    del w
    rope = F.DeviceRope(cfg, T, dev)
    ws = F.workspace(cfg, T, T, dev)
    e_all = torch.from_numpy(synth.context_embeddings(p, seed, order)).to(dev, bf)
    k_pre = torch.zeros((T, kvd), dtype=bf, device=dev)
    v_pre = torch.zeros((T, kvd), dtype=bf, device=dev)
    for c in range(p.n_chunks):
        lo, hi = int(offs[c]), int(offs[c + 1])
        L = hi - lo
        h_iso = torch.empty((L, d), dtype=bf, device=dev)
        kt = torch.empty((L, kvd), dtype=bf, device=dev)
        vt = torch.empty((L, kvd), dtype=bf, device=dev)
        F.full_prefill_layer(cfg, layer, rope, e_all[lo:hi].contiguous(), L, 0, kt, vt, h_iso, ws)
        h2 = torch.empty_like(h_iso)
        F.full_prefill_layer(cfg, layer, rope, h_iso, L, 0, k_pre[lo:hi], v_pre[lo:hi], h2, ws)
    h_full = torch.empty((T, d), dtype=bf, device=dev)
    kf = torch.empty((T, kvd), dtype=bf, device=dev)
    vf = torch.empty((T, kvd), dtype=bf, device=dev)
    F.full_prefill_layer(cfg, layer, rope, e_all, T, 0, kf, vf, h_full, ws)
    # select call: recompute all candidates once, keep the HKVD set S
    k_cache = k_pre.clone()
    v_cache = v_pre.clone()
    F.rope_shift(cfg, rope, k_cache, T * kvd, 1, T, offs)
    s_all = torch.arange(L0, T, dtype=torch.int32, device=dev)
    m_sel = F.expected_m_out(T, n_ctx, T - L0, k)
    s_sel = torch.empty(m_sel, dtype=torch.int32, device=dev)
    h_sel = torch.empty((m_sel, d), dtype=bf, device=dev)
    dv_all = torch.empty(T - L0, dtype=torch.float32, device=dev)
    F.blend_layer(cfg, layer, rope, k_cache, v_cache, T, n_ctx, L0, s_all, T - L0, h_full, s_all, k, h_sel, dv_all,
                  s_sel, ws)
    torch.cuda.synchronize()
    S = s_sel.clone()
    m = m_sel
    hout = torch.empty((m, d), dtype=bf, device=dev)
    s_out = torch.empty(m, dtype=torch.int32, device=dev)
    dv = torch.empty(m, dtype=torch.float32, device=dev)
    # the step works on its own copy of the precomputed cache; repeated steps
    # rotate the same rows again and rewrite the same recomputed rows, at
    # identical cost
    kb = k_pre.clone()
    vb = v_pre.clone()

    def step():
        if args.separate_shift:
            F.rope_shift(cfg, rope, kb, T * kvd, 1, T, offs)
            F.blend_layer(cfg, layer, rope, kb, vb, T, n_ctx, L0, S, m, h_full, S, k, hout, dv, s_out, ws)
        else:
            F.blend_layer_realign(cfg, layer, rope, kb, vb, T, offs, S, m, h_full, S, k, hout, dv, s_out, ws)

    if args.calib_copy:
        src = torch.ones(CALIB_COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"set-up done (k={k}, m={m}); timing {args.steps} steps after {args.warmup} warm-up steps")
    # ---------------- timed region ----------------
    for _ in range(args.warmup):
        step()
    # one hipEvent pair per step on the stream the library launches on (torch's
    # current stream); the step time is the median of the per-step times
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    ms = float(np.median(step_ms))
    ms_wall = (t1 - t0) * 1e3 / args.steps

    # per-kernel durations: the same steps again with hipEvents around every launch
    F.profile_begin()
    for _ in range(args.steps):
        step()
    stats = F.profile_end()
    torch.cuda.synchronize()
    positions = s_out.cpu().numpy()
    flops = layer_flops(p, m, m, positions)
    kern = {}
    for name, st in stats.items():
        avg = st["total_ms"] / st["launches"]
        e = {"avg_ms": round(avg, 5), "launches_per_step": st["launches"] // args.steps}
        if name in flops:
            tf = flops[name] / (avg * 1e-3) / 1e12
            e.update({"tflops": round(tf, 1), "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4)})
        kern[name] = e
    shift_bytes = 2 * n_cand * kvd * 2
    if "rope_shift" in kern:
        gbs = shift_bytes / (kern["rope_shift"]["avg_ms"] * 1e-3) / 1e9
        kern["rope_shift"].update({"gbs": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
    dom = "gemm_gateup"
    dom_ms = kern[dom]["avg_ms"]
    dom_tf = flops[dom] / (dom_ms * 1e-3) / 1e12
    total_flops = sum(flops.values())

    extra = {}
    if args.extra:
        # select call (recompute all candidates + top-k) and full prefill of the same layer
        kk, vv = k_cache.clone(), v_cache.clone()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            F.blend_layer(cfg, layer, rope, kk, vv, T, n_ctx, L0, s_all, T - L0, h_full, s_all, k, h_sel, dv_all,
                          s_sel, ws)
        torch.cuda.synchronize()
        extra["select_call_ms"] = round((time.perf_counter() - t0) * 100, 4)
        h2 = torch.empty((T, d), dtype=bf, device=dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            F.full_prefill_layer(cfg, layer, rope, h_full, T, 0, kf, vf, h2, ws)
        torch.cuda.synchronize()
        extra["full_prefill_ms"] = round((time.perf_counter() - t0) * 100, 4)
        extra.update(hbm_kernels_measure())

    if args.batch > 1:
        # n_req requests of the same shape (own caches, same rows): one shift
        # launch over all their caches + one batched layer
        nb = args.batch
        kvb = k_pre.unsqueeze(0).repeat(nb, 1, 1).contiguous()
        vvb = v_pre.unsqueeze(0).repeat(nb, 1, 1).contiguous()
        reqs = [dict(k_cache=kvb[i], v_cache=vvb[i], T=T, n_ctx=n_ctx, first_chunk_len=L0, m_in=m, k_out=k)
                for i in range(nb)]
        s_cat = S.repeat(nb).contiguous()
        h_cat = h_full[S.long()].repeat(nb, 1).contiguous()
        yb = torch.empty((nb * m, d), dtype=bf, device=dev)
        dvb = torch.empty(nb * m, dtype=torch.float32, device=dev)
        sob = torch.empty(nb * m, dtype=torch.int32, device=dev)
        wsb = F.workspace(cfg, T, nb * m, dev)

        def bstep():
            F.rope_shift(cfg, rope, kvb, T * kvd, nb, T, offs)
            F.blend_batch(cfg, layer, rope, reqs, s_cat, h_cat, yb, dvb, sob, wsb)

        for _ in range(args.warmup):
            bstep()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            bstep()
        torch.cuda.synchronize()
        bms = (time.perf_counter() - t0) * 1e3 / args.steps
        F.profile_begin()
        for _ in range(args.steps):
            bstep()
        bstats = F.profile_end()
        torch.cuda.synchronize()
        bflops = {kname: v * nb for kname, v in flops.items()}
        bk = {}
        for name, st in bstats.items():
            avg = st["total_ms"] / st["launches"]
            e = {"avg_ms": round(avg, 5)}
            if name in bflops:
                e["frac_mfma"] = round(bflops[name] / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
            bk[name] = e
        extra["batch"] = {"n_req": nb, "ms_per_step": round(bms, 5), "tokens_per_s": round(nb * T / (bms * 1e-3), 1),
                          "speedup_vs_single_steps": round(nb * ms / bms, 3),
                          "layer_frac_mfma": round(total_flops * nb / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "kernels": bk}
    if args.pipeline:
        extra["pipeline"] = pipeline_measure(seed)
    if args.analytics:
        extra["analytics"] = analytics_measure(seed)
    if args.llama70b:
        extra["llama70b_layer"] = layer70b_measure(seed, args.steps)
    if args.sweep:
        extra["sweep"] = sweep_measure(seed, min(args.steps, 20))
    if args.fp8:
        extra["fp8"] = fp8_measure(p, m, args.steps)
        # the same step with the layer's projections in 8 bits (cb_blend_layer_fp8)
        layer8 = F.DeviceLayerFp8.quantized(cfg, layer)
        ws8 = F.workspace_fp8(cfg, T, T, dev)
        kb8, vb8 = k_pre.clone(), v_pre.clone()

        def step8():
            F.rope_shift(cfg, rope, kb8, T * kvd, 1, T, offs)
            F.blend_layer_fp8(cfg, layer8, rope, kb8, vb8, T, n_ctx, L0, S, m, h_full, S, k, hout, dv, s_out, ws8)

        for _ in range(args.warmup):
            step8()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step8()
        torch.cuda.synchronize()
        ms8 = (time.perf_counter() - t0) * 1e3 / args.steps
        F.profile_begin()
        for _ in range(args.steps):
            step8()
        st8 = F.profile_end()
        torch.cuda.synchronize()
        extra["fp8"]["layer"] = {
            "ms_per_step": round(ms8, 5), "tokens_per_s": round(T / (ms8 * 1e-3), 1),
            "speedup_vs_bf16": round(ms / ms8, 3),
            "kernels": {n: {"avg_ms": round(v["total_ms"] / v["launches"], 5),
                            "launches_per_step": v["launches"] // args.steps} for n, v in st8.items()}}
        del layer8, ws8, kb8, vb8

    cpu = None
    log(f"gpu timing done: {ms:.4f} ms/step")
    if not args.no_cpu:
        log("timing the CPU oracle")
        cpu = cpu_baseline(p, seed, k, args.cpu_seconds)
        if args.cpu_extra:
            log("timing the CPU oracle on the other workloads")
            cpu["extra"] = cpu_extra_measure(seed)

    out = {
        "metric": "blended-context tokens/s at r=0.15 (Llama-8B-shaped layer)",
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_mean_wall": round(ms_wall, 5),
        "ms_per_step_min_max": [round(float(step_ms.min()), 5), round(float(step_ms.max()), 5)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) embeddings; cached KV from isolated prefill)",
        "config": {"workload": "llama8b_layer: 6x512-token chunks + 32-token query (T=3104), r=0.15, "
                               "k=461 HKVD + 32 query rows; d=4096, 32q/8kv heads x128, ffn 14336",
                   "T": T, "k": k, "m": m, "step": "cb_rope_shift + cb_blend_layer" if args.separate_shift else "cb_blend_layer_realign",
                   "weights": "bf16; W_gate/W_up repacked and the attention RMSNorm gain folded into W_qkv "
                              "once at load time (cb_pack_gateup, cb_fold_qkv; untimed)"},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(dom_tf, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(dom_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(dom),
                     "flops_per_launch": flops[dom]},
        "layer_tflops": round(total_flops / (ms * 1e-3) / 1e12, 1),
        "layer_frac_mfma": round(total_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "kernels": kern,
        "cpu_baseline": cpu,
    }
    out.update(extra)
    print(json.dumps(out))


def copy_cold_measure(reps=6, nbytes=1 << 30):
    """cb_stream_copy (the library's streaming copy: 16-byte accesses, 1 KB
    of contiguous memory per wave instruction, non-temporal stores) of 1 GiB,
    rotating over four 1 GiB buffers so that no call finds its data in the
    256 MB Infinity Cache; hipMemcpy's device-to-device copy beside it.
    Bytes moved = read + write = 2 GiB per call."""
    import torch
    from rag_kv_cache_layer_amd import fusor as F
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(4)]
    for b in bufs:
        b.fill_(1)
    F.stream_copy(bufs[0], bufs[1])
    torch.cuda.synchronize()

    def med(fn):
        times = []
        for i in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn(i)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return sorted(times)[len(times) // 2]
    ms = med(lambda i: F.stream_copy(bufs[(2 * i) % 4], bufs[(2 * i + 1) % 4]))
    ms_d2d = med(lambda i: bufs[(2 * i + 1) % 4].copy_(bufs[(2 * i) % 4]))
    del bufs
    torch.cuda.empty_cache()
    return {"bytes": 2 * nbytes, "ms": round(ms, 4), "gbs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(2 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "hipmemcpy_d2d_gbs": round(2 * nbytes / (ms_d2d * 1e-3) / 1e9, 1)}


def hbm_kernels_measure():
    """Cold, large launches of the bandwidth-bound kernels, each with its rate
    as a fraction of the 8 TB/s peak and of the streaming copy's rate."""
    out = {"copy_cold": copy_cold_measure()}
    ceiling = out["copy_cold"]["gbs"]
    out["shift_stack"] = shift_stack_measure()
    out["kdev_cold"] = kdev_cold_measure()
    out["kv_expand_stack"] = kv_expand_measure()
    for k in ("shift_stack", "kdev_cold", "kv_expand_stack"):
        out[k]["frac_of_copy"] = round(out[k]["gbs"] / ceiling, 4)
    return out


def shift_stack_measure(reps=6):
    """cb_rope_shift over a whole 32-layer 8B stack's key cache (8 x 512 + 64
    tokens: 3584 shifted rows per layer), one launch per call, alternating
    between two caches of 272 MB each so that no call finds its data in the
    256 MB Infinity Cache.  Algorithmic bytes: every shifted element is read
    and written once."""
    import torch
    from rag_kv_cache_layer_amd import fusor as F
    from rag_kv_cache_layer_amd import synth
    p = synth.PRESETS["llama8b_stack"]
    cfg = F.config_of(p)
    offs = synth.chunk_offsets(p, range(p.n_chunks))
    T, kvd, L = p.T, p.kv_dim, p.n_layers
    rope = F.DeviceRope(cfg, T)
    bufs = [torch.randn((L, T, kvd), device="cuda").to(torch.bfloat16) for _ in range(2)]
    F.rope_shift(cfg, rope, bufs[0], T * kvd, L, T, offs)
    torch.cuda.synchronize()
    times = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        F.rope_shift(cfg, rope, bufs[i % 2], T * kvd, L, T, offs)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    nbytes = 2 * L * (p.n_ctx - int(offs[1])) * kvd * 2
    # reference: a device-to-device copy moving the same bytes (read + write)
    src = bufs[0].view(-1)[: nbytes // 4]
    dst = bufs[1].view(-1)[: nbytes // 4]
    ctimes = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ctimes.append(e0.elapsed_time(e1))
    cms = sorted(ctimes)[len(ctimes) // 2]
    return {"layers": L, "bytes": nbytes, "ms": round(ms, 4), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "copy_same_bytes_gbs": round(nbytes / (cms * 1e-3) / 1e9, 1)}


def kdev_cold_measure(reps=6):
    """The standalone K deviation of cb_select_hkvd (k_new given) over the
    candidates of the 8B layer with 32 chunks x 512 + 64 tokens (15872 rows of
    8 KV heads x 128): each call reads the new K rows and the cached K rows
    (65 MB), rotating over four sets of buffers (260 MB) so that no call finds
    its data in the 256 MB Infinity Cache.  The kernel's own time comes from
    the library's per-launch events ("kdev"); the top-k of the same call is
    reported beside it."""
    import torch
    from rag_kv_cache_layer_amd import fusor as F
    from rag_kv_cache_layer_amd import synth
    p = synth.sweep_preset(32, 1500)
    cfg = F.config_of(p)
    T, kvd = p.T, p.kv_dim
    L0 = 512
    n = p.n_ctx - L0
    k = F.num_selected(1500, p.n_ctx, n)
    rows = torch.arange(L0, L0 + n, dtype=torch.int32, device="cuda")
    sets = [(torch.randn((n, kvd), device="cuda").to(torch.bfloat16),
             torch.randn((T, kvd), device="cuda").to(torch.bfloat16)) for _ in range(4)]
    dv = torch.empty(n, dtype=torch.float32, device="cuda")
    so = torch.empty(k, dtype=torch.int32, device="cuda")
    ws = F.workspace(cfg, T, T)
    F.select_hkvd(cfg, sets[0][0], sets[0][1], T, rows, n, k, dv, so, ws)
    torch.cuda.synchronize()
    F.profile_begin()
    for i in range(reps):
        F.select_hkvd(cfg, sets[(i + 1) % 4][0], sets[(i + 1) % 4][1], T, rows, n, k, dv, so, ws)
    torch.cuda.synchronize()
    st = F.profile_end()
    kd = st["kdev"]
    ms = kd["total_ms"] / kd["launches"]
    nbytes = 2 * n * kvd * 2
    out = {"rows": n, "bytes": nbytes, "ms": round(ms, 4), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    if "select_topk" in st:
        out["topk_ms"] = round(st["select_topk"]["total_ms"] / st["select_topk"]["launches"], 4)
    return out


def sweep_measure(seed, steps):
    """The 8B-shaped layer over n x 512 context tokens + 64 query tokens (chunk
    order permuted), n = 4, 16, 32, at recompute ratios r = 0.05 .. 1: for each
    point the select call (untimed) picks S, then the step on S
    (cb_blend_layer_realign: re-alignment + blend call) is timed, next to a
    full prefill of the same layer over all T rows (the full KV recompute
    baseline).  Seeded N(0, 0.02) weights drawn on the device (W_gate/W_up
    packed and the attention RMSNorm folded into W_qkv, as for the 8B step),
    seeded N(0, 1) cached K/V and layer inputs."""
    import torch
    from rag_kv_cache_layer_amd import fusor as F
    from rag_kv_cache_layer_amd import synth
    base = synth.sweep_preset(4, 1500)
    cfg = F.config_of(base)
    g = torch.Generator(device="cuda")
    g.manual_seed(3000 + seed)
    shapes = {"w_q": (base.q_dim, base.d_model), "w_k": (base.kv_dim, base.d_model),
              "w_v": (base.kv_dim, base.d_model), "w_o": (base.d_model, base.q_dim),
              "w_gate": (base.ffn_dim, base.d_model), "w_up": (base.ffn_dim, base.d_model),
              "w_down": (base.d_model, base.ffn_dim)}
    w = {n: (torch.randn(s, generator=g, device="cuda") * 0.02).to(torch.bfloat16) for n, s in shapes.items()}
    w["attn_norm"] = torch.ones(base.d_model, device="cuda")
    w["mlp_norm"] = torch.ones(base.d_model, device="cuda")
    layer = F.DeviceLayer(cfg, w).pack_gateup().fold_qkv()
    del w

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    out = []
    for n_chunks in (4, 16, 32):
        p = synth.sweep_preset(n_chunks, 1500)
        T, n_ctx, kvd, d = p.T, p.n_ctx, p.kv_dim, p.d_model
        offs = synth.chunk_offsets(p, synth.chunk_order(p, seed))
        L0 = int(offs[1])
        rope = F.DeviceRope(cfg, T)
        ws = F.workspace(cfg, T, T)
        k_pre = torch.randn((T, kvd), generator=g, device="cuda").to(torch.bfloat16)
        v_pre = torch.randn((T, kvd), generator=g, device="cuda").to(torch.bfloat16)
        x = torch.randn((T, d), generator=g, device="cuda").to(torch.bfloat16)
        kf, vf = torch.empty_like(k_pre), torch.empty_like(v_pre)
        yf = torch.empty_like(x)
        t_full = timed(lambda: F.full_prefill_layer(cfg, layer, rope, x, T, 0, kf, vf, yf, ws), max(steps // 4, 2))
        s_all = torch.arange(L0, T, dtype=torch.int32, device="cuda")
        dv = torch.empty(T - L0, dtype=torch.float32, device="cuda")
        for r_e4 in (500, 1000, 1500, 3000, 10000):
            k = F.num_selected(r_e4, n_ctx, n_ctx - L0)
            m = F.expected_m_out(T, n_ctx, T - L0, k)
            S = torch.empty(m, dtype=torch.int32, device="cuda")
            hout = torch.empty((m, d), dtype=torch.bfloat16, device="cuda")
            kc, vc = k_pre.clone(), v_pre.clone()
            F.rope_shift(cfg, rope, kc, T * kvd, 1, T, offs)
            F.blend_layer(cfg, layer, rope, kc, vc, T, n_ctx, L0, s_all, T - L0, x, s_all, k, hout, dv, S, ws)
            torch.cuda.synchronize()
            so = torch.empty(m, dtype=torch.int32, device="cuda")
            kb, vb = k_pre.clone(), v_pre.clone()

            def step():
                F.blend_layer_realign(cfg, layer, rope, kb, vb, T, offs, S, m, x, S, k, hout, dv, so, ws)

            ms = timed(step, steps)
            out.append({"chunks": n_chunks, "T": T, "r": r_e4 / 1e4, "k": k, "ms": round(ms, 4),
                        "tokens_per_s": round(T / (ms * 1e-3), 1), "full_prefill_ms": round(t_full, 4),
                        "speedup_vs_full_prefill": round(t_full / ms, 2)})
            del S, hout, kc, vc, so, kb, vb
        del ws, k_pre, v_pre, x, kf, vf, yf, rope
        torch.cuda.empty_cache()
    return out


def layer70b_measure(seed, steps):
    """The blend call of one 70B-shaped layer (d 8192, 64/8 heads x 128, FFN
    28672; 8 x 500 + 32 tokens, r = 0.15) with seeded N(0, 0.02) weights drawn
    on the device, seeded N(0, 1) cached K/V and layer inputs: the select call
    once (untimed) for the kept set, then the step on that set
    (cb_blend_layer_realign, weights packed and folded), as for the 8B layer."""
    import torch
    from rag_kv_cache_layer_amd import fusor as F
    from rag_kv_cache_layer_amd import synth
    p = synth.PRESETS["llama70b_stack"]
    cfg = F.config_of(p)
    g = torch.Generator(device="cuda")
    g.manual_seed(2000 + seed)
    shapes = {"w_q": (p.q_dim, p.d_model), "w_k": (p.kv_dim, p.d_model), "w_v": (p.kv_dim, p.d_model),
              "w_o": (p.d_model, p.q_dim), "w_gate": (p.ffn_dim, p.d_model), "w_up": (p.ffn_dim, p.d_model),
              "w_down": (p.d_model, p.ffn_dim)}
    w = {n: (torch.randn(s, generator=g, device="cuda") * 0.02).to(torch.bfloat16) for n, s in shapes.items()}
    w["attn_norm"] = torch.ones(p.d_model, device="cuda")
    w["mlp_norm"] = torch.ones(p.d_model, device="cuda")
    layer = F.DeviceLayer(cfg, w).pack_gateup().fold_qkv()
    del w
    T, n_ctx, kvd, d = p.T, p.n_ctx, p.kv_dim, p.d_model
    offs = synth.chunk_offsets(p, range(p.n_chunks))
    L0 = int(offs[1])
    k = F.num_selected(p.r_e4, n_ctx, n_ctx - L0)
    rope = F.DeviceRope(cfg, T)
    ws = F.workspace(cfg, T, T)
    k_pre = torch.randn((T, kvd), generator=g, device="cuda").to(torch.bfloat16)
    v_pre = torch.randn((T, kvd), generator=g, device="cuda").to(torch.bfloat16)
    x = torch.randn((T, d), generator=g, device="cuda").to(torch.bfloat16)
    kc, vc = k_pre.clone(), v_pre.clone()
    F.rope_shift(cfg, rope, kc, T * kvd, 1, T, offs)
    s_all = torch.arange(L0, T, dtype=torch.int32, device="cuda")
    m = F.expected_m_out(T, n_ctx, T - L0, k)
    S = torch.empty(m, dtype=torch.int32, device="cuda")
    hout = torch.empty((m, d), dtype=torch.bfloat16, device="cuda")
    dv = torch.empty(T - L0, dtype=torch.float32, device="cuda")
    F.blend_layer(cfg, layer, rope, kc, vc, T, n_ctx, L0, s_all, T - L0, x, s_all, k, hout, dv, S, ws)
    torch.cuda.synchronize()
    so = torch.empty(m, dtype=torch.int32, device="cuda")
    kb, vb = k_pre.clone(), v_pre.clone()

    def step():
        F.blend_layer_realign(cfg, layer, rope, kb, vb, T, offs, S, m, x, S, k, hout, dv, so, ws)

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    F.profile_begin()
    for _ in range(steps):
        step()
    st = F.profile_end()
    torch.cuda.synchronize()
    flops = layer_flops(p, m, m, so.cpu().numpy())
    kern = {}
    for name, e in st.items():
        avg = e["total_ms"] / e["launches"]
        kern[name] = {"avg_ms": round(avg, 5)}
        if name in flops:
            kern[name]["frac_mfma"] = round(flops[name] / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    total = sum(flops.values())
    return {"workload": "llama70b_layer: 8x500-token chunks + 32-token query (T=4032), r=0.15, "
                        f"k={k} + 32 query rows; d=8192, 64q/8kv heads x128, ffn 28672",
            "ms_per_step": round(ms, 5), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "layer_tflops": round(total / (ms * 1e-3) / 1e12, 1),
            "layer_frac_mfma": round(total / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "kernels": kern}


def kv_expand_measure(reps=6):
    """cb_kv_from_fp8 over a whole 32-layer 8B stack (8 x 512 + 64 tokens):
    8-bit K and V codes of every row expanded into bf16 caches with the keys
    re-aligned, one launch, alternating between two destination pairs so that
    no call finds its data in the Infinity Cache.  Algorithmic bytes: codes
    and exponents read once, the bf16 caches written once."""
    import torch
    from rag_kv_cache_layer_amd import fusor as F
    from rag_kv_cache_layer_amd import synth
    p = synth.PRESETS["llama8b_stack"]
    cfg = F.config_of(p)
    offs = synth.chunk_offsets(p, range(p.n_chunks))
    T, kvd, L, H = p.T, p.kv_dim, p.n_layers, p.n_kv_heads
    rope = F.DeviceRope(cfg, T)
    codes = [torch.randint(0, 0x7E, (L, T, kvd), dtype=torch.uint8, device="cuda") for _ in range(2)]
    exps = [torch.randint(-12, 4, (L, T, H), dtype=torch.int32, device="cuda") for _ in range(2)]
    dsts = [[torch.empty((L, T, kvd), dtype=torch.bfloat16, device="cuda") for _ in range(2)] for _ in range(2)]
    run = lambda i: F.kv_from_fp8(cfg, rope, codes[0], exps[0], codes[1], exps[1], dsts[i % 2][0], dsts[i % 2][1],
                                  T * kvd, L, T, offs)
    run(0)
    torch.cuda.synchronize()
    times = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run(i + 1)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    nbytes = 2 * L * T * (kvd + H * 4) + 2 * L * T * kvd * 2
    return {"layers": L, "rows": T, "bytes": nbytes, "ms": round(ms, 4),
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def pipeline_measure(seed, reps=3):
    """The 32-layer 8B-shaped stack (8 x 512 + 64 tokens, r 0.30 -> 0.15) with
    every layer's chunk KV in pinned host memory (CacheBlend section 5): the
    time to load all layers alone (copy stream), to recompute with the KV
    already resident, and both pipelined by cb_blend_stack; plus the loading
    controller's ratio from the measured link rate and full-prefill time.
    Weights are seeded N(0, 0.02) drawn on the device (14 GB)."""
    import torch
    from rag_kv_cache_layer_amd import fusor as F
    from rag_kv_cache_layer_amd import synth
    p = synth.PRESETS["llama8b_stack"]
    cfg = F.config_of(p)
    log("pipeline: generating the 32-layer stack on the device")
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 + seed)
    shapes = {"w_q": (p.q_dim, p.d_model), "w_k": (p.kv_dim, p.d_model), "w_v": (p.kv_dim, p.d_model),
              "w_o": (p.d_model, p.q_dim), "w_gate": (p.ffn_dim, p.d_model), "w_up": (p.ffn_dim, p.d_model),
              "w_down": (p.d_model, p.ffn_dim)}
    layers = []
    for _ in range(p.n_layers):
        w = {n: (torch.randn(s, generator=g, device="cuda") * 0.02).to(torch.bfloat16) for n, s in shapes.items()}
        w["attn_norm"] = torch.ones(p.d_model, device="cuda")
        w["mlp_norm"] = torch.ones(p.d_model, device="cuda")
        layers.append(F.DeviceLayer(cfg, w))
        del w
    T, n_ctx = p.T, p.n_ctx
    offs = synth.chunk_offsets(p, range(p.n_chunks))
    L0 = int(offs[1])
    shape = (p.n_layers, T, p.n_kv_heads, p.head_dim)
    Kh = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16).cpu().pin_memory()
    Vh = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16).cpu().pin_memory()
    x0 = torch.randn((T - L0, p.d_model), generator=g, device="cuda").to(torch.bfloat16)
    ks = F.filter_schedule(p.n_layers, 3000, 1500, n_ctx, n_ctx - L0)
    rope = F.DeviceRope(cfg, T)
    wss = torch.empty(F.stack_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    K = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    V = torch.empty_like(K)
    cs = torch.cuda.Stream()
    kv_bytes = 2 * K.numel() * 2

    def timed(fn):
        best = None
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            best = dt if best is None else min(best, dt)
        return best

    def load():
        with torch.cuda.stream(cs):
            K.copy_(Kh, non_blocking=True)
            V.copy_(Vh, non_blocking=True)

    def resident():
        F.blend_stack_native(cfg, layers, rope, K, V, T, offs, x0, ks, wss)

    def streamed():
        F.blend_stack_native(cfg, layers, rope, K, V, T, offs, x0, ks, wss, k_src=Kh, v_src=Vh, copy_stream=cs)

    log("pipeline: timing")
    t_load = timed(load)
    t_comp = timed(resident)    # align + recompute with the KV already in device memory
    t_pipe = timed(streamed)    # load each layer (copy stream) + align + recompute (compute stream)
    # the same KV stored as 8-bit codes with one exponent per (token, KV head):
    # half the bytes over the link, expanded (and re-aligned) on the device
    q8 = []
    for X in (K, V):
        X.copy_(Kh if X is K else Vh)
        c, e = F.quantize_fp8(X.view(-1, p.head_dim))
        q8 += [c.view(shape).cpu().pin_memory(), e.view(shape[:3]).cpu().pin_memory()]
    torch.cuda.synchronize()
    kc8, ke8, vc8, ve8 = q8
    d8 = [torch.empty(t.shape, dtype=t.dtype, device="cuda") for t in q8]
    kv8_bytes = sum(t.numel() * t.element_size() for t in q8)

    def load8():
        with torch.cuda.stream(cs):
            for d_, s_ in zip(d8, q8):
                d_.copy_(s_, non_blocking=True)

    def streamed8():
        F.blend_stack_native(cfg, layers, rope, K, V, T, offs, x0, ks, wss, k_src=kc8, v_src=vc8,
                             k_src_exp=ke8, v_src_exp=ve8, copy_stream=cs)

    t_load8 = timed(load8)
    t_pipe8 = timed(streamed8)
    # one full-prefill layer over the context, for the controller's recompute estimate
    h_in = torch.randn((T, p.d_model), generator=g, device="cuda").to(torch.bfloat16)
    h_out = torch.empty_like(h_in)
    kf = torch.empty((T, p.kv_dim), dtype=torch.bfloat16, device="cuda")
    vf = torch.empty_like(kf)
    ws1 = F.workspace(cfg, T, T)
    t_pf = timed(lambda: F.full_prefill_layer(cfg, layers[0], rope, h_in, T, 0, kf, vf, h_out, ws1))
    link = kv_bytes / t_load                          # bytes per second over PCIe
    kv_token = 2 * p.kv_dim * 2                       # one layer's K and V per token, bf16
    r_e4 = F.pick_ratio(t_pf * 1e6, kv_token, T, link * 1e-6, 1500)
    return {"workload": "llama8b_stack: 32 layers, 8x512-token chunks + 64-token query (T=4160), r 0.30 -> 0.15",
            "kv_bytes": kv_bytes, "load_ms": round(t_load * 1e3, 3), "recompute_ms": round(t_comp * 1e3, 3),
            "pipelined_ms": round(t_pipe * 1e3, 3), "link_gbs": round(link / 1e9, 2),
            "hidden_fraction": round((t_load + t_comp - t_pipe) / min(t_load, t_comp), 3),
            "pcie_inclusive_tokens_per_s": round(T / t_pipe, 1),
            "full_prefill_layer_ms": round(t_pf * 1e3, 4), "controller_r_e4": r_e4,
            "kv8": {"kv_bytes": kv8_bytes, "load_ms": round(t_load8 * 1e3, 3),
                    "pipelined_ms": round(t_pipe8 * 1e3, 3),
                    "hidden_fraction": round((t_load8 + t_comp - t_pipe8) / min(t_load8, t_comp), 3),
                    "pcie_inclusive_tokens_per_s": round(T / t_pipe8, 1),
                    "controller_r_e4": F.pick_ratio(t_pf * 1e6, kv8_bytes / (p.n_layers * T), T, link * 1e-6,
                                                    1500)}}


def analytics_measure(seed):
    """Deviation analytics of the 32-layer 8B stack (8 x 512 + 64 tokens) with
    seeded N(0, 0.02) weights drawn on the device and N(0, 1) embeddings; the
    chunk caches come from each chunk's isolated prefill through the stack."""
    import torch
    from rag_kv_cache_layer_amd import analytics as GA
    from rag_kv_cache_layer_amd import fusor as F
    from rag_kv_cache_layer_amd import synth
    p = synth.PRESETS["llama8b_stack"]
    cfg = F.config_of(p)
    log("analytics: generating the 32-layer stack on the device")
    g = torch.Generator(device="cuda")
    g.manual_seed(2000 + seed)
    shapes = {"w_q": (p.q_dim, p.d_model), "w_k": (p.kv_dim, p.d_model), "w_v": (p.kv_dim, p.d_model),
              "w_o": (p.d_model, p.q_dim), "w_gate": (p.ffn_dim, p.d_model), "w_up": (p.ffn_dim, p.d_model),
              "w_down": (p.d_model, p.ffn_dim)}
    layers = []
    for _ in range(p.n_layers):
        w = {n: (torch.randn(s, generator=g, device="cuda") * 0.02).to(torch.bfloat16) for n, s in shapes.items()}
        w["attn_norm"] = torch.ones(p.d_model, device="cuda")
        w["mlp_norm"] = torch.ones(p.d_model, device="cuda")
        layers.append(F.DeviceLayer(cfg, w))
        del w
    offs = synth.chunk_offsets(p, range(p.n_chunks))
    x_all = torch.randn((p.T, p.d_model), generator=g, device="cuda").to(torch.bfloat16)
    rope = F.DeviceRope(cfg, p.T)
    t0 = time.perf_counter()
    out = GA.stack_study(cfg, layers, rope, x_all, offs, [0, 500, 1000, 1500, 3000, 10000])
    torch.cuda.synchronize()
    ts = out["top_share"]
    return {"workload": "llama8b_stack: 32 layers, 8x512-token chunks + 64-token query (T=4160)",
            "ratios": [r / 1e4 for r in out["ratios_e4"]],
            "attn_dev_rel_mean": [round(x, 6) for x in out["attn_dev_mean"]],
            "top_share_mean_layers_1plus": {f: round(sum(v[1:]) / (len(v) - 1), 4) for f, v in ts.items()},
            "spearman_neighbours_mean": round(sum(out["spearman_neighbours"]) / len(out["spearman_neighbours"]), 4),
            "spearman_neighbours_min": round(min(out["spearman_neighbours"]), 4),
            "seconds": round(time.perf_counter() - t0, 2)}


PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 matrix peak


def fp8_measure(p, m, steps):
    """The four projections of the 8B layer at m rows with fp8 E4M3 operands:
    weights quantized once (untimed), each activation matrix quantized per
    row inside the timed call (cb_quantize_fp8 + cb_gemm_fp8, bf16 out)."""
    import torch
    from rag_kv_cache_layer_amd import fusor as F
    d, q, kv, ffn = p.d_model, p.q_dim, p.kv_dim, p.ffn_dim
    g = torch.Generator(device="cuda")
    g.manual_seed(3000)
    shapes = {"qkv": (q + 2 * kv, d), "o": (d, q), "gateup": (2 * ffn, d), "down": (d, ffn)}
    out = {}
    for name, (N, K) in shapes.items():
        w = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        qw, ew = F.quantize_fp8(w)
        del w
        x = torch.randn((m, K), generator=g, device="cuda").to(torch.bfloat16)
        qx = torch.empty((m, K), dtype=torch.uint8, device="cuda")
        ex = torch.empty(m, dtype=torch.int32, device="cuda")
        y = torch.empty((m, N), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(int(F.lib().cb_gemm_fp8_workspace_size(m, N, K)), 1), dtype=torch.uint8, device="cuda")

        def call():
            F.quantize_fp8(x, qx, ex)
            F.gemm_fp8(qx, ex, qw, ew, y, ws)

        for _ in range(5):
            call()
        F.profile_begin()
        for _ in range(steps):
            call()
        st = F.profile_end()
        torch.cuda.synchronize()
        # 128x128 kernel (+ split-K sum) or the 256x256 kernel for wide outputs
        gm = sum(st[k]["total_ms"] / st[k]["launches"] for k in ("gemm_fp8", "gemm_fp8_big", "gemm_fp8_split_sum")
                 if k in st)
        qm = st["quantize_fp8"]["total_ms"] / st["quantize_fp8"]["launches"]
        tf = 2 * m * N * K / (gm * 1e-3) / 1e12
        out[name] = {"gemm_ms": round(gm, 5), "quantize_ms": round(qm, 5), "tflops": round(tf, 1),
                     "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)}
        del qw, ew, x, qx, y, ws
    return out


def cpu_baseline(p, seed, k, budget_s):
    """The oracle's blend call (numpy fp32) on the host cores, same shapes."""
    from threadpoolctl import threadpool_info

    from oracle import blend
    from rag_kv_cache_layer_amd import synth
    T, n_ctx = p.T, p.n_ctx
    L0 = p.chunk_lens[0]
    w = synth.layer_weights(p, seed, 0)
    K = synth.random_normal(p, seed, (T, p.n_kv_heads, p.head_dim), tag_layer=11)
    V = synth.random_normal(p, seed, (T, p.n_kv_heads, p.head_dim), tag_layer=12)
    x = synth.random_normal(p, seed, (T, p.d_model), tag_layer=13)
    S = np.concatenate([synth.random_subset(p, seed, L0, n_ctx, k), np.arange(n_ctx, T)]).astype(np.int64)
    times = []
    t_start = time.perf_counter()
    while not times or (time.perf_counter() - t_start < budget_s and len(times) < 20):
        t0 = time.perf_counter()
        blend.blend_layer(w, p, K, V, n_ctx, S, x[S], k, store="bf16")
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(T / t, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(times)} oracle blend calls (numpy fp32, {threads} BLAS threads) of the same layer "
                      f"and shapes, median {t * 1e3:.0f} ms"}


def cpu_extra_measure(seed, reps=3):
    """The oracle (numpy fp32, the host's BLAS threads unless stated) on the
    other workloads, median of `reps` calls (one call for the large layers):
    blend call = selective recompute of k candidates + the query at ratio r;
    full prefill = the same layer over all T rows.  Stack figures are one
    layer's time times the layer count (an estimate, labelled so)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import blend, layer
    from rag_kv_cache_layer_amd import synth

    def med(f, n):
        ts = []
        for _ in range(n):
            t0 = time.perf_counter()
            f()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    def case(p, k, n_rep):
        T, n_ctx = p.T, p.n_ctx
        L0 = p.chunk_lens[0]
        w = synth.layer_weights(p, seed, 0)
        K = synth.random_normal(p, seed, (T, p.n_kv_heads, p.head_dim), tag_layer=11)
        V = synth.random_normal(p, seed, (T, p.n_kv_heads, p.head_dim), tag_layer=12)
        x = synth.random_normal(p, seed, (T, p.d_model), tag_layer=13)
        S = np.concatenate([synth.random_subset(p, seed, L0, n_ctx, min(k, n_ctx - L0)),
                            np.arange(n_ctx, T)]).astype(np.int64)
        st = "bf16" if p.dtype == "bf16" else None
        return (lambda: blend.blend_layer(w, p, K, V, n_ctx, S, x[S], k, store=st),
                lambda: layer.full_prefill(w, x, p, 0, store=st))

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    out = {"threads": threads}
    tiny = synth.PRESETS["tiny_f32"]
    kt = blend.num_selected(tiny.r_e4, tiny.n_ctx, tiny.n_ctx - tiny.chunk_lens[0])
    bl, fp = case(tiny, kt, 1)
    out["tiny_f32"] = {"T": tiny.T, "k": kt, "blend_ms": round(med(bl, 7) * 1e3, 3),
                       "full_prefill_ms": round(med(fp, 7) * 1e3, 3)}
    with threadpool_limits(1):
        out["tiny_f32"]["blend_ms_1thread"] = round(med(bl, 7) * 1e3, 3)
        out["tiny_f32"]["full_prefill_ms_1thread"] = round(med(fp, 7) * 1e3, 3)
    log("cpu extra: tiny done")
    p8 = synth.PRESETS["llama8b_layer"]
    k8 = blend.num_selected(p8.r_e4, p8.n_ctx, p8.n_ctx - p8.chunk_lens[0])
    _, fp = case(p8, k8, 1)
    out["llama8b_layer"] = {"T": p8.T, "full_prefill_ms": round(med(fp, 1) * 1e3, 1)}
    log("cpu extra: 8B full prefill done")
    sw = synth.sweep_preset(4, 1500)
    res = {"T": sw.T}
    for r_e4 in (1500, 10000):
        k = blend.num_selected(r_e4, sw.n_ctx, sw.n_ctx - sw.chunk_lens[0])
        bl, fp = case(sw, k, reps)
        res[f"blend_ms_r{r_e4 / 1e4:g}"] = round(med(bl, reps) * 1e3, 1)
    res["full_prefill_ms"] = round(med(fp, 1) * 1e3, 1)
    out["sweep_4_chunks"] = res
    log("cpu extra: sweep done")
    st = synth.PRESETS["llama8b_stack"]
    ks = blend.filter_schedule(st.n_layers, st.r_e4, st.r_last_e4, st.n_ctx, st.n_ctx - st.chunk_lens[0])
    k_mean = int(round(float(np.mean(ks))))
    bl, _ = case(st, k_mean, 1)
    t = med(bl, 1)
    out["llama8b_stack"] = {"T": st.T, "layers": st.n_layers, "k_mean": k_mean, "layer_ms": round(t * 1e3, 1),
                            "stack_ms_estimate": round(t * 1e3 * st.n_layers, 0)}
    log("cpu extra: 8B stack spot layer done")
    p70 = synth.PRESETS["llama70b_stack"]
    k70 = blend.num_selected(p70.r_e4, p70.n_ctx, p70.n_ctx - p70.chunk_lens[0])
    bl, fp = case(p70, k70, 1)
    log("cpu extra: 70B inputs ready")
    tb = med(bl, 1)
    log("cpu extra: 70B blend layer done")
    tf = med(fp, 1)
    out["llama70b_stack"] = {"T": p70.T, "layers": p70.n_layers, "k": k70, "blend_layer_ms": round(tb * 1e3, 1),
                             "full_prefill_layer_ms": round(tf * 1e3, 1),
                             "blend_stack_ms_estimate": round(tb * 1e3 * p70.n_layers, 0),
                             "full_prefill_stack_ms_estimate": round(tf * 1e3 * p70.n_layers, 0)}
    log("cpu extra: 70B spot layers done")
    return out


if __name__ == "__main__":
    main()
