#!/usr/bin/env python3
"""Benchmark of the ZGCM-1 attention core on one MI355X.

Headline workload: the full 32-layer attention schedule (27 gated-SWA layers, global causal layers at
6, 12, 18, 24, 30) prefilling one 16,384-token sequence, 32 query / 8 KV heads of dim 128, window 128,
RoPE on 42 dims with base 10,000, seeded N(0,1) bf16 q/k/v/gate per layer.  One step = the 32 layer
calls.  Metric: attention tokens/s (16,384 / step time) and the global-layer kernel against the MFMA
roofline.

Second workload ("decode"): one hybrid decode step of 32 sequences, each at position 262,144, through all
32 layers: the 5 global layers read full bf16 KV caches (262,144 cached positions x 8 KV heads x 128) and
the 27 SWA layers their 128-slot rings; cache contents and new q/k/v/gate ~N(0,1), RoPE base 1e7.
Metric: tokens/s (32 / step time), and the split-K decode kernel against the HBM roofline.

Inputs are generated on the GPU before the timed region.  The CPU baseline times the fp64 oracle on a
bounded sample of the prefill workload (see cpu_baseline.sample in the output).

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-decode] [--no-cpu-baseline]
       python bench.py --schedule-sweep   (per-layer times at 4K..256K composed into 5:1, 3:1, 1:1, all-global)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA, TFLOP/s
GLOBAL_LAYERS = (6, 12, 18, 24, 30)
N_LAYERS, HQ, HKV, D, W, R = 32, 32, 8, 128, 128, 42


def stored_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, or None when
    the kernel's source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic_prefill_16k_decode_256k.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        f = line.split()
        if len(f) == 5 and f[0] == "traffic" and f[1] == kernel:
            kv = dict(x.split("=", 1) for x in f[2:])
            src = os.path.join(ROOT, kv["source"])
            if os.path.exists(src) and hashlib.sha256(open(src, "rb").read()).hexdigest() == kv["sha256"]:
                return int(kv["bytes"])
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sync():
    import torch
    torch.cuda.synchronize()


# ------------------------------------------------------------------------------------------ prefill
def setup_prefill(seed=1003, S=16384, B=1):
    import torch
    import synth
    layers = []
    for l in range(1, N_LAYERS + 1):
        glob = l in GLOBAL_LAYERS
        t = {}
        for name, tid, H in (("q", synth.TENSOR_Q, HQ), ("k", synth.TENSOR_K, HKV), ("v", synth.TENSOR_V, HKV)) + \
                (() if glob else (("gate", synth.TENSOR_GATE, HQ),)):
            t[name] = synth.normal_bf16_device(seed, l, tid, (B, S, H, D))
        for name, tid in (("wq", synth.TENSOR_WQ), ("wk", synth.TENSOR_WK)):
            bits = synth.norm_weight_bf16(seed, l, tid, D)
            t[name] = torch.from_numpy(bits.view("int16")).cuda().view(torch.bfloat16)
        t["out"] = torch.empty((B, S, HQ, D), dtype=torch.bfloat16, device="cuda")
        t["glob"] = glob
        layers.append(t)
    import global_attention_gated_amd as zg
    ws = torch.empty(zg.workspace_bytes(B, S, HKV, D), dtype=torch.uint8, device="cuda")
    sync()
    return layers, ws


def prefill_step(zg, layers, ws):
    for t in layers:
        if t["glob"]:
            zg.global_prefill(t["q"], t["k"], t["v"], t["wq"], t["wk"], t["out"], rotary_dims=R, rope_base=1e4,
                              eps=1e-6, workspace=ws)
        else:
            zg.swa_prefill(t["q"], t["k"], t["v"], t["gate"], t["wq"], t["wk"], t["out"], window=W, rotary_dims=R,
                           rope_base=1e4, eps=1e-6, workspace=ws)


def run_prefill(zg, steps, warmup, S=16384, B=1):
    layers, ws = setup_prefill(S=S, B=B)
    for _ in range(warmup):
        prefill_step(zg, layers, ws)
    sync()
    # Timed steps: only the roofline kernel (the global layer's attention) records events, so the step time
    # carries the cost of 10 events per step, not of 74.  The other kernels' durations come from a short pass
    # after the timed steps, with every kernel timed.
    zg.kernel_timer_enable(True, only="attn_global")
    sync()
    t0 = time.perf_counter()
    for _ in range(steps):
        prefill_step(zg, layers, ws)
    sync()
    t1 = time.perf_counter()
    kt = {"attn_global": zg.kernel_timer_read("attn_global")}
    zg.kernel_timer_enable(True)
    for _ in range(min(steps, 3)):
        prefill_step(zg, layers, ws)
    sync()
    kt.update({n: zg.kernel_timer_read(n) for n in ("attn_swa", "kv_stage")})
    zg.kernel_timer_enable(False)
    ms = (t1 - t0) * 1e3 / steps
    pairs_global = S * (S + 1) // 2
    flop_global = 4 * D * HQ * B * pairs_global                       # per launch (one global layer)
    pairs_swa = sum(min(i + 1, W) for i in range(S))
    flop_swa = 4 * D * HQ * B * pairs_swa
    bytes_swa = B * S * (3 * HQ * D * 2 + 2 * HKV * D * 2)             # q, gate, out + k, v (bf16)
    bytes_stage = B * S * HKV * D * 2 * 4                              # k, v in (bf16); k_hat, v^T out (fp16)
    total_flop = 5 * flop_global + 27 * flop_swa
    g_ms, g_n = kt["attn_global"]
    s_ms, s_n = kt["attn_swa"]
    p_ms, p_n = kt["kv_stage"]
    g_avg = g_ms / max(g_n, 1)
    s_avg = s_ms / max(s_n, 1)
    res = {
        "ms_per_step": ms,
        "tokens_per_s": B * S / (ms / 1e3),
        "schedule_tflops": total_flop / (ms / 1e3) / 1e12,
        "schedule_mfma_frac": total_flop / (ms / 1e3) / 1e12 / MFMA_PEAK_TFLOPS,
        "kernels": {
            "attn_global": {"avg_ms": g_avg, "launches": g_n, "algorithmic_tflop_per_launch": flop_global / 1e12,
                            "tflops": flop_global / (g_avg / 1e3) / 1e12},
            "attn_swa": {"avg_ms": s_avg, "launches": s_n, "algorithmic_bytes_per_launch": bytes_swa,
                         "gbs": bytes_swa / (s_avg / 1e3) / 1e9,
                         "hbm_frac": bytes_swa / (s_avg / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": stored_traffic("attn_swa"),
                         "tflops": flop_swa / (s_avg / 1e3) / 1e12},
            "kv_stage": {"avg_ms": p_ms / max(p_n, 1), "launches": p_n,
                         "algorithmic_bytes_per_launch": bytes_stage,
                         "gbs": bytes_stage / (p_ms / max(p_n, 1) / 1e3) / 1e9 if p_n else None},
            "timing": "attn_global: HIP events over the timed steps; attn_swa, kv_stage: HIP events over a "
                      "pass of up to 3 steps right after them",
        },
        "roofline": {"bound": "mfma", "achieved": flop_global / (g_avg / 1e3) / 1e12, "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": flop_global / (g_avg / 1e3) / 1e12 / MFMA_PEAK_TFLOPS,
                     "traffic": stored_traffic("attn_global"),
                     "kernel": "attn_pp_kernel<false> (one global layer per launch)"},
    }
    del layers, ws
    import torch
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------------------ decode
def fill_cache(zg, cache, seed, P):
    """Cache contents ~N(0,1) in the cache layout, as if positions 0..P-1 had been written."""
    import synth
    for l in range(1, cache.n_layers + 1):
        kp, vp, slots = cache.layer_view(l)
        synth.fill_kv_cache_layer(kp, vp, slots, seed=seed, layer=l, batch=cache.batch, n_kv_heads=HKV, head_dim=D,
                                  n_positions=P, is_global=l in cache.global_layers, window=W)
        for b in range(cache.batch):
            cache.set_length(l, b, P)


def run_decode(zg, steps, warmup, B=32, P=262144, seed=1004):
    import torch
    import synth
    cache = zg.KVCache(n_layers=N_LAYERS, global_layers=GLOBAL_LAYERS, batch=B, n_kv_heads=HKV, head_dim=D, window=W,
                       max_tokens=P + 1)
    fill_cache(zg, cache, seed, P)
    q = synth.normal_bf16_device(seed, 1000, synth.TENSOR_Q, (N_LAYERS, B, HQ, D))
    k = synth.normal_bf16_device(seed, 1000, synth.TENSOR_K, (N_LAYERS, B, HKV, D))
    v = synth.normal_bf16_device(seed, 1000, synth.TENSOR_V, (N_LAYERS, B, HKV, D))
    g = synth.normal_bf16_device(seed, 1000, synth.TENSOR_GATE, (N_LAYERS, B, HQ, D))
    import numpy as np
    wq = np.stack([synth.norm_weight_bf16(seed, l, synth.TENSOR_WQ, D) for l in range(1, N_LAYERS + 1)])
    wk = np.stack([synth.norm_weight_bf16(seed, l, synth.TENSOR_WK, D) for l in range(1, N_LAYERS + 1)])
    wq = torch.from_numpy(wq.view(np.int16)).cuda().view(torch.bfloat16)
    wk = torch.from_numpy(wk.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty_like(q)
    positions = [P] * B
    sync()

    def step():
        zg.hybrid_decode_step(q, k, v, g, wq, wk, positions, cache, out, rotary_dims=R, rope_base=1e7, eps=1e-6)
        for l in range(1, N_LAYERS + 1):       # host-side: back to P cached positions (rewriting row P is idempotent)
            for b in range(B):
                cache.set_length(l, b, P)

    for _ in range(warmup):
        step()
    sync()
    zg.kernel_timer_enable(True)
    sync()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    sync()
    t1 = time.perf_counter()
    kt = {n: zg.kernel_timer_read(n) for n in ("decode_global", "decode_swa", "decode_append", "decode_merge")}
    zg.kernel_timer_enable(False)
    ms = (t1 - t0) * 1e3 / steps
    keys = P + 1
    glob_bytes = 5 * B * HKV * keys * D * 2 * 2                        # K and V rows read per launch
    swa_bytes = 27 * B * HKV * W * D * 2 * 2
    io_bytes = N_LAYERS * B * (3 * HQ * D * 2 + 2 * HKV * D * 2)        # q, gate, out, k, v of the new token
    step_bytes = glob_bytes + swa_bytes + io_bytes
    g_ms, g_n = kt["decode_global"]
    g_avg = g_ms / max(g_n, 1)
    res = {
        "ms_per_step": ms,
        "tokens_per_s": B / (ms / 1e3),
        "step_bytes": step_bytes,
        "step_gbs": step_bytes / (ms / 1e3) / 1e9,
        "step_hbm_frac": step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "kv_cache_device_bytes": cache.device_bytes,
        "kernels": {n: {"avg_ms": t / max(c, 1), "launches": c} for n, (t, c) in kt.items()},
        "roofline": {"bound": "hbm", "achieved": glob_bytes / (g_avg / 1e3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": glob_bytes / (g_avg / 1e3) / 1e9 / HBM_PEAK_GBS, "traffic": stored_traffic("decode_global"),
                     "kernel": "decode_attn_kernel<global split-K> (5 global layers per launch)",
                     "algorithmic_bytes_per_launch": glob_bytes},
        "config": {"workload": "hybrid decode step, 32 seqs at position 262144, 32 layers (27 SWA ring + 5 global)",
                   "batch": B, "position": P, "layers": N_LAYERS, "global_layers": list(GLOBAL_LAYERS), "q_heads": HQ,
                   "kv_heads": HKV, "head_dim": D, "window": W, "rotary_dims": R, "rope_base": 1e7, "seed": seed},
    }
    cache.close()
    del q, k, v, g, out
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------------------ schedule sweep
SCHEDULES = ("5:1", "3:1", "1:1", "all-global")


def schedule_globals(name: str, n_layers: int = N_LAYERS):
    """1-based global layers of a 32-layer stack.  "5:1" is the pages' placement (one global layer after every
    five gated-SWA layers: 6, 12, ..., 30); "3:1" and "1:1" put one after every three or every one SWA layer;
    "all-global" is full attention everywhere."""
    period = {"5:1": 6, "3:1": 4, "1:1": 2, "all-global": 1}[name]
    return tuple(l for l in range(1, n_layers + 1) if l % period == 0)


def compose_schedules(per_layer_ms, footprint):
    """Attention time of one prefill pass through the 32-layer stack for each schedule, from measured
    per-layer times {S: {"swa": ms, "global": ms}} (layers of one kind cost the same at one length);
    footprint(S, globals) gives the KV-cache bytes."""
    out = {}
    for name in SCHEDULES:
        g = schedule_globals(name)
        rows = []
        for S in sorted(per_layer_ms):
            t = per_layer_ms[S]
            ms = (N_LAYERS - len(g)) * t["swa"] + len(g) * t["global"]
            rows.append({"seq_len": S, "attention_ms": ms, "tokens_per_s": S / (ms / 1e3),
                         "kv_cache_bytes": footprint(S, g)})
        out[name] = {"global_layers": list(g), "n_global": len(g), "by_length": rows}
    ref = {r["seq_len"]: r["attention_ms"] for r in out["all-global"]["by_length"]}
    for name in SCHEDULES:
        for r, rg in zip(out[name]["by_length"], out["all-global"]["by_length"]):
            r["speedup_vs_all_global"] = ref[r["seq_len"]] / r["attention_ms"]
            r["kv_ratio_all_global"] = rg["kv_cache_bytes"] / r["kv_cache_bytes"]
    return out


def run_schedule_sweep(zg, lengths=(4096, 16384, 65536, 262144), reps=3, seed=1006):
    """Per-layer prefill time of one gated-SWA and one global layer (batch 1, 32q/8kv, D 128, W 128, R 42) at
    each length, median of `reps` HIP-event timings after one warm-up call, composed into the schedules."""
    import statistics
    import torch
    import synth
    per_layer = {}
    for S in lengths:
        t = {n: synth.normal_bf16_device(seed, 1, tid, (1, S, H, D)) for n, tid, H in
             (("q", synth.TENSOR_Q, HQ), ("k", synth.TENSOR_K, HKV), ("v", synth.TENSOR_V, HKV),
              ("gate", synth.TENSOR_GATE, HQ))}
        wq, wk = (torch.from_numpy(synth.norm_weight_bf16(seed, 1, tid, D).view("int16")).cuda().view(torch.bfloat16)
                  for tid in (synth.TENSOR_WQ, synth.TENSOR_WK))
        out = torch.empty_like(t["q"])
        ws = torch.empty(zg.workspace_bytes(1, S, HKV, D), dtype=torch.uint8, device="cuda")
        base = 1e4 if S <= 16384 else 1e7

        def swa():
            zg.swa_prefill(t["q"], t["k"], t["v"], t["gate"], wq, wk, out, window=W, rotary_dims=R, rope_base=base,
                           eps=1e-6, workspace=ws)

        def glob():
            zg.global_prefill(t["q"], t["k"], t["v"], wq, wk, out, rotary_dims=R, rope_base=base, eps=1e-6,
                              workspace=ws)

        per_layer[S] = {}
        for name, fn in (("swa", swa), ("global", glob)):
            fn()
            sync()
            ms = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                e1.synchronize()
                ms.append(e0.elapsed_time(e1))
            per_layer[S][name] = statistics.median(ms)
        log(f"sweep: S={S}: SWA layer {per_layer[S]['swa']:.3f} ms, global layer {per_layer[S]['global']:.3f} ms")
        del t, out, ws
        torch.cuda.empty_cache()
    sched = compose_schedules(per_layer, lambda S, g: zg.footprint_bytes(S, global_layers=g))
    return per_layer, sched


# ------------------------------------------------------------------------------------------ whole layers
D_MODEL = 4096


def run_layers(zg, steps=5, warmup=2, S=16384, seed=1007):
    """One gated-SWA and one global layer from the hidden state (q/k/v(/g) projections, attention core, o_proj),
    batch 1 x S tokens, d_model 4096, 32q/8kv, random-init weights N(0,1)/sqrt(fan_in); HIP-event time per
    layer call and the hipBLASLt GEMM time within it (kernel timer "linear")."""
    import numpy as np
    import torch
    import synth

    def weight(tensor, n_out, n_in):
        w = synth.normal_bf16_device(seed, 0, tensor, (n_out, n_in))
        return (w.float() / float(np.sqrt(n_in))).to(torch.bfloat16)   # power-of-two scale: exact

    h = synth.normal_bf16_device(seed, 0, synth.TENSOR_H, (1, S, D_MODEL))
    w = {"q": weight(synth.TENSOR_PQ, HQ * D, D_MODEL), "k": weight(synth.TENSOR_PK, HKV * D, D_MODEL),
         "v": weight(synth.TENSOR_PV, HKV * D, D_MODEL), "g": weight(synth.TENSOR_PG, HQ * D, D_MODEL),
         "o": weight(synth.TENSOR_PO, D_MODEL, HQ * D)}
    nw = torch.from_numpy(synth.norm_weight_bf16(seed, 1, synth.TENSOR_WQ, D).view("int16")).cuda().view(torch.bfloat16)
    y = torch.empty_like(h)
    ws = torch.empty(zg.fp8_layer_workspace_bytes(1, S, D_MODEL, HQ, HKV, D), dtype=torch.uint8, device="cuda")
    f8 = {"gated_swa_layer_fp8": zg.Fp8Layer(D_MODEL, HQ, HKV, D), "global_layer_fp8": zg.Fp8Layer(D_MODEL, HQ, HKV, D)}
    calls = {
        "gated_swa_layer": lambda: zg.gated_swa_layer(h, w["q"], w["k"], w["v"], w["g"], w["o"], nw, nw, y, Hq=HQ,
                                                      Hkv=HKV, window=W, rotary_dims=R, rope_base=1e4, workspace=ws),
        "global_layer": lambda: zg.global_layer(h, w["q"], w["k"], w["v"], w["o"], nw, nw, y, Hq=HQ, Hkv=HKV,
                                                rotary_dims=R, rope_base=1e4, workspace=ws),
        "gated_swa_layer_fp8": lambda: zg.gated_swa_layer_fp8(
            h, w["q"], w["k"], w["v"], w["g"], w["o"], nw, nw, y, fp8=f8["gated_swa_layer_fp8"], Hq=HQ, Hkv=HKV,
            window=W, rotary_dims=R, rope_base=1e4, workspace=ws),
        "global_layer_fp8": lambda: zg.global_layer_fp8(
            h, w["q"], w["k"], w["v"], w["o"], nw, nw, y, fp8=f8["global_layer_fp8"], Hq=HQ, Hkv=HKV, rotary_dims=R,
            rope_base=1e4, workspace=ws),
    }
    gemm_flop = {"gated_swa_layer": 2 * S * D_MODEL * (3 * HQ * D + 2 * HKV * D),
                 "global_layer": 2 * S * D_MODEL * (2 * HQ * D + 2 * HKV * D)}
    gemm_flop["gated_swa_layer_fp8"], gemm_flop["global_layer_fp8"] = gemm_flop["gated_swa_layer"], gemm_flop["global_layer"]
    res = {}
    for name, fn in calls.items():
        for _ in range(warmup):
            fn()
        sync()
        zg.kernel_timer_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        sync()
        lin_ms, lin_n = zg.kernel_timer_read("linear")
        q_ms, _ = zg.kernel_timer_read("fp8_quantize")
        zg.kernel_timer_enable(False)
        ms = e0.elapsed_time(e1) / steps
        gms = lin_ms / steps
        peak = MFMA_PEAK_TFLOPS * (2 if name.endswith("_fp8") else 1)        # dense fp8 MFMA: 5.0 PFLOP/s
        res[name] = {"ms_per_layer": ms, "gemm_ms_per_layer": gms, "gemm_launches_per_layer": lin_n // steps,
                     "quantize_ms_per_layer": q_ms / steps, "gemm_tflop_per_layer": gemm_flop[name] / 1e12,
                     "gemm_tflops": gemm_flop[name] / (gms / 1e3) / 1e12, "gemm_peak_tflops": peak,
                     "gemm_mfma_frac": gemm_flop[name] / (gms / 1e3) / 1e12 / peak}
        log(f"layers: {name}: {ms:.3f} ms/layer, GEMMs {gms:.3f} ms ({res[name]['gemm_tflops']:.0f} TFLOP/s), "
            f"quantise {q_ms / steps:.3f} ms")
    for sfx in ("", "_fp8"):
        stack_ms = 27 * res["gated_swa_layer" + sfx]["ms_per_layer"] + 5 * res["global_layer" + sfx]["ms_per_layer"]
        res["stack" + sfx] = {"ms": stack_ms, "tokens_per_s": S / (stack_ms / 1e3)}
        log(f"layers: 27 gated + 5 global{sfx or ' (bf16)'}: {stack_ms:.2f} ms, {S / (stack_ms / 1e3):.0f} tokens/s")
    for st in f8.values():
        st.close()

    # one 4096 -> 4096 projection of the S tokens: bf16 against FP8 with delayed scaling (quantisation of x and
    # W, GEMM and scale update all inside the timed call)
    x, wq = h.view(S, D_MODEL), w["q"]
    fp8 = zg.Fp8Linear(D_MODEL, HQ * D)
    yp = torch.empty((S, HQ * D), dtype=torch.bfloat16, device="cuda")
    flop = 2 * S * D_MODEL * HQ * D
    for name, fn in (("bf16", lambda: zg.linear_bf16(x, wq, yp)), ("fp8_delayed", lambda: fp8(x, wq, yp))):
        for _ in range(warmup):
            fn()
        sync()
        zg.kernel_timer_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        sync()
        g_ms, _ = zg.kernel_timer_read("linear")
        q_ms, _ = zg.kernel_timer_read("fp8_quantize")
        zg.kernel_timer_enable(False)
        ms = e0.elapsed_time(e1) / steps
        peak = MFMA_PEAK_TFLOPS * (2 if name == "fp8_delayed" else 1)        # dense fp8 MFMA: 5.0 PFLOP/s
        res.setdefault("projection_4096x4096", {"tokens": S, "tflop": flop / 1e12})[name] = {
            "ms": ms, "gemm_ms": g_ms / steps, "quantize_ms": q_ms / steps, "tflops": flop / (ms / 1e3) / 1e12,
            "gemm_tflops": flop / (g_ms / steps / 1e3) / 1e12, "gemm_peak_tflops": peak,
            "gemm_frac": flop / (g_ms / steps / 1e3) / 1e12 / peak}
        log(f"layers: projection {name}: {ms:.3f} ms (GEMM {g_ms / steps:.3f} ms, "
            f"{flop / (g_ms / steps / 1e3) / 1e12:.0f} TFLOP/s; quantise {q_ms / steps:.3f} ms)")
    fp8.close()
    del h, w, y, ws, x, yp
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------------------ training backward
def run_backward(zg, steps=5, warmup=2, S=16384, seed=1008):
    """Training forward (with lse) and backward of one gated-SWA and one global layer, batch 1 x S tokens, 32q/8kv:
    HIP-event time of each call and of each backward kernel family.  The global backward's algorithmic work is
    2.5x the forward's (S, dP, dV, dQ, dK: 5 x 2D flop per visible (head, key) pair); the kernels execute 3.5x
    (S and dP are formed in both the dK/dV and the dQ kernel)."""
    import numpy as np
    import torch
    import synth
    res = {}
    for name, gated, layer in (("gated_swa", True, 1), ("global", False, 6)):
        q = synth.normal_bf16_device(seed, layer, synth.TENSOR_Q, (1, S, HQ, D))
        k = synth.normal_bf16_device(seed, layer, synth.TENSOR_K, (1, S, HKV, D))
        v = synth.normal_bf16_device(seed, layer, synth.TENSOR_V, (1, S, HKV, D))
        g = synth.normal_bf16_device(seed, layer, synth.TENSOR_GATE, (1, S, HQ, D)) if gated else None
        dout = synth.normal_bf16_device(seed, layer, synth.TENSOR_DOUT, (1, S, HQ, D))
        wq = torch.from_numpy(synth.norm_weight_bf16(seed, layer, synth.TENSOR_WQ, D).view("int16")).cuda().view(torch.bfloat16)
        wk = torch.from_numpy(synth.norm_weight_bf16(seed, layer, synth.TENSOR_WK, D).view("int16")).cuda().view(torch.bfloat16)
        out = torch.empty_like(q)
        lse = torch.empty((1, HQ, S), dtype=torch.float32, device="cuda")
        fws = torch.empty(zg.workspace_bytes(1, S, HKV, D), dtype=torch.uint8, device="cuda")
        bws = torch.empty(zg.backward_workspace_bytes(1, S, HQ, HKV, D), dtype=torch.uint8, device="cuda")
        grads = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
                 "dq_norm_w": torch.empty(D, dtype=torch.float32, device="cuda"),
                 "dk_norm_w": torch.empty(D, dtype=torch.float32, device="cuda")}
        if gated:
            grads["dgate"] = torch.empty_like(g)

        def fwd():
            zg.prefill_train(q, k, v, g, wq, wk, window=W, rotary_dims=R, rope_base=1e4, out=out, lse=lse, workspace=fws)

        def bwd():
            zg.prefill_backward(q, k, v, g, wq, wk, out, lse, dout, window=W, rotary_dims=R, rope_base=1e4,
                                grads=grads, workspace=bws)

        times = {}
        for tag, fn in (("forward", fwd), ("backward", bwd)):
            for _ in range(warmup):
                fn()
            sync()
            zg.kernel_timer_enable(True)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            sync()
            times[tag] = e0.elapsed_time(e1) / steps
            if tag == "backward":
                times["kernels"] = {kn: zg.kernel_timer_read(kn)[0] / steps for kn in ("bwd_prep", "bwd_kv", "bwd_q")}
            zg.kernel_timer_enable(False)
        pairs = S * (S + 1) // 2 if not gated else sum(min(i + 1, W) for i in range(S))
        fwd_flop = 4 * D * HQ * pairs
        r = {"forward_ms": times["forward"], "backward_ms": times["backward"], "backward_kernels_ms": times["kernels"],
             "forward_tflop": fwd_flop / 1e12, "backward_algorithmic_tflop": 2.5 * fwd_flop / 1e12,
             "backward_tflops": 2.5 * fwd_flop / (times["backward"] / 1e3) / 1e12}
        mm = times["kernels"]["bwd_kv"] + times["kernels"]["bwd_q"]
        r["mfma_kernels_tflops"] = 2.5 * fwd_flop / (mm / 1e3) / 1e12
        r["mfma_kernels_frac"] = r["mfma_kernels_tflops"] / MFMA_PEAK_TFLOPS
        res[name] = r
        log(f"backward: {name}: forward {times['forward']:.3f} ms, backward {times['backward']:.3f} ms "
            f"(prep {times['kernels']['bwd_prep']:.3f}, dK/dV {times['kernels']['bwd_kv']:.3f}, "
            f"dQ {times['kernels']['bwd_q']:.3f}; norm/RoPE backward in the dK and dQ epilogues); "
            f"{r['backward_tflops']:.0f} TFLOP/s algorithmic, dK/dV + dQ kernels {r['mfma_kernels_tflops']:.0f} TFLOP/s")
        del q, k, v, g, dout, out, lse, fws, bws, grads
        torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------------------ chunked prefill
def run_chunked(zg, S_total=262144, C=16384, seed=1005, passes=1):
    """Long-context chunked prefill: one sequence of S_total tokens in C-token chunks through the 32-layer schedule
    against a KV cache (RoPE base 1e7).  Each chunk's 32 layer inputs are generated before its timed layer calls;
    the time is the sum over chunks of HIP-event times around the 32 calls of a chunk.  The global layers' tile
    kernel is timed on its own too (kernel timer), for its roofline line."""
    import torch
    import synth
    cache = zg.KVCache(n_layers=N_LAYERS, global_layers=GLOBAL_LAYERS, batch=1, n_kv_heads=HKV, head_dim=D, window=W,
                       max_tokens=S_total)
    ws = torch.empty(zg.workspace_bytes(1, C, HKV, D, pos0=S_total - C), dtype=torch.uint8, device="cuda")
    w = {}
    for l in range(1, N_LAYERS + 1):
        for name, tid in (("wq", synth.TENSOR_WQ), ("wk", synth.TENSOR_WK)):
            w[(l, name)] = torch.from_numpy(synth.norm_weight_bf16(seed, l, tid, D).view("int16")).cuda().view(torch.bfloat16)
    out = torch.empty((1, C, HQ, D), dtype=torch.bfloat16, device="cuda")
    total_ms, chunk_ms = 0.0, []
    glob_ms, glob_n, glob_flop = 0.0, 0, 0
    for p in range(passes):
        if p:
            for l in range(1, N_LAYERS + 1):
                cache.set_length(l, 0, 0)
        for c in range(S_total // C):
            pos0 = c * C
            t = []
            for l in range(1, N_LAYERS + 1):
                glob = l in GLOBAL_LAYERS
                d = {}
                for name, tid, H in (("q", synth.TENSOR_Q, HQ), ("k", synth.TENSOR_K, HKV), ("v", synth.TENSOR_V, HKV)) + \
                        (() if glob else (("gate", synth.TENSOR_GATE, HQ),)):
                    d[name] = synth.normal_bf16_device(seed, l, tid, (1, C, H, D), index_offset=pos0 * H * D)
                t.append(d)
            sync()
            zg.kernel_timer_enable(True, only="attn_global")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for l in range(1, N_LAYERS + 1):
                d = t[l - 1]
                if l in GLOBAL_LAYERS:
                    zg.global_prefill(d["q"], d["k"], d["v"], w[(l, "wq")], w[(l, "wk")], out, rotary_dims=R,
                                      rope_base=1e7, eps=1e-6, pos0=pos0, cache=cache, layer=l, workspace=ws)
                else:
                    zg.swa_prefill(d["q"], d["k"], d["v"], d["gate"], w[(l, "wq")], w[(l, "wk")], out, window=W,
                                   rotary_dims=R, rope_base=1e7, eps=1e-6, pos0=pos0, cache=cache, layer=l,
                                   workspace=ws)
            e1.record()
            sync()
            ms = e0.elapsed_time(e1)
            gms, gn = zg.kernel_timer_read("attn_global")
            zg.kernel_timer_enable(False)
            if p == passes - 1:
                chunk_ms.append(ms)
                total_ms += ms
                glob_ms += gms
                glob_n += gn
                glob_flop += 5 * 4 * D * HQ * (C * pos0 + C * (C + 1) // 2)
            log(f"chunked: pass {p} chunk {c} at {pos0}: {ms:.1f} ms (global kernels {gms:.1f} ms)")
            del t
    fp = zg.footprint_bytes(S_total)
    fp_all = zg.footprint_bytes(S_total, global_layers=range(1, N_LAYERS + 1))
    res = {
        "ms_total": total_ms,
        "tokens_per_s": S_total / (total_ms / 1e3),
        "chunk_ms": chunk_ms,
        "global_kernel": {"ms_total": glob_ms, "launches": glob_n, "algorithmic_tflop": glob_flop / 1e12,
                          "tflops": glob_flop / (glob_ms / 1e3) / 1e12},
        "roofline": {"bound": "mfma", "achieved": glob_flop / (glob_ms / 1e3) / 1e12, "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": glob_flop / (glob_ms / 1e3) / 1e12 / MFMA_PEAK_TFLOPS, "traffic": None,
                     "kernel": "attn_pp_kernel<false> over all 16 chunks of the 5 global layers"},
        "kv_cache_bytes": {"hybrid": fp, "all_global": fp_all, "hybrid_gib": fp / 2**30, "all_global_gib": fp_all / 2**30,
                           "device_bytes": cache.device_bytes},
    }
    cache.close()
    del ws
    import torch as _t
    _t.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------------------ CPU baseline
def cpu_baseline(S=16384, n_rows=8192, seed=1003):
    """The fp64 oracle on a sample of the prefill workload: n_rows random positions, all 32 query heads, in
    one gated-SWA layer (layer 1) and one global layer (layer 6).  Per-token time = 27 x (SWA row time +
    SWA key-prologue time / S) + 5 x (global row time + global key-prologue time / S).  Input generation
    is not timed."""
    import numpy as np
    import oracle
    import synth
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(S, size=n_rows, replace=False))
    per_layer = {}
    for layer, glob in ((1, False), (6, True)):
        k = synth.normal_bf16(seed, layer, synth.TENSOR_K, (1, S, HKV, D))[0]
        v = synth.normal_bf16(seed, layer, synth.TENSOR_V, (1, S, HKV, D))[0]
        wq = synth.norm_weight_bf16(seed, layer, synth.TENSOR_WQ, D)
        wk = synth.norm_weight_bf16(seed, layer, synth.TENSOR_WK, D)
        qidx = (rows[:, None, None] * HQ * D + np.arange(HQ)[None, :, None] * D + np.arange(D)[None, None, :])
        q = synth.normal_bf16_at(seed, layer, synth.TENSOR_Q, qidx)              # [n_rows, HQ, D]
        gate = None if glob else synth.normal_bf16_at(seed, layer, synth.TENSOR_GATE, qidx)
        pos = np.arange(S)
        t0 = time.perf_counter()
        khat = oracle.cache_key(oracle.qk_prologue(k, pos[:, None], wk, 1e-6, R, 1e4))     # [S, HKV, D]
        t1 = time.perf_counter()
        qhat = oracle.qk_prologue(q, rows[:, None], wq, 1e-6, R, 1e4)
        vf = oracle.bf16_to_f64(v)
        G = HQ // HKV
        if glob:
            hi = int(rows.max()) + 1
            for h in range(HQ):
                oracle.attend(qhat[:, h], rows, khat[:hi, h // G], vf[:hi, h // G], pos[:hi], None)
        else:
            # blocks of 32 consecutive sampled rows, each block over the keys its rows' windows span (about 190
            # for 32 rows of a 2-in-4 sample), the G heads of a KV head at once
            for i0 in range(0, n_rows, 32):
                rb = rows[i0:i0 + 32]
                lo, hi = max(0, int(rb[0]) - W + 1), int(rb[-1]) + 1
                for kh in range(HKV):
                    hs = slice(kh * G, (kh + 1) * G)
                    oracle.attend(qhat[i0:i0 + 32, hs].reshape(-1, D), np.repeat(rb, G), khat[lo:hi, kh],
                                  vf[lo:hi, kh], pos[lo:hi], W, gate[i0:i0 + 32, hs].reshape(-1, D))
        t2 = time.perf_counter()
        per_layer["global" if glob else "swa"] = ((t2 - t1) / n_rows, (t1 - t0) / S)
    per_tok = 27 * sum(per_layer["swa"]) + 5 * sum(per_layer["global"])
    return {"value": 1.0 / per_tok, "unit": "tokens/s", "cores": oracle.num_threads(), "host_cores": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{n_rows} random positions x 32 heads of layer 1 (gated SWA) and layer 6 (global) of the "
                      f"1x16384 schedule, plus each layer's key prologue over all {S} positions; scaled to one "
                      f"token through 27 SWA + 5 global layers",
            "seconds": None}


# ------------------------------------------------------------------------------------------ main
def run_gemm_ceiling(shapes=((8192, 8192, 8192), (16384, 16384, 8192), (16384, 8192, 16384)), calls=20, warmup=5):
    """What a vendor library's dense fp16 GEMM (torch.matmul on hipBLASLt) reaches on this GPU: the practical
    ceiling that power sets for MFMA-dense work, the context of the attention kernel's MFMA fraction."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(0)
    out = []
    for M, N, K in shapes:
        a = torch.randn(M, K, device="cuda", dtype=torch.float16, generator=gen)
        b = torch.randn(K, N, device="cuda", dtype=torch.float16, generator=gen)
        for _ in range(warmup):
            c = a @ b
        sync()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(calls):
            c = a @ b
        e1.record()
        sync()
        ms = e0.elapsed_time(e1) / calls
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        log(f"gemm: fp16 {M}x{N}x{K} {ms:.3f} ms, {tf:.0f} TFLOP/s = {tf / MFMA_PEAK_TFLOPS:.3f} of the peak")
        out.append({"M": M, "N": N, "K": K, "ms": ms, "tflops": tf, "frac": tf / MFMA_PEAK_TFLOPS})
        del a, b, c
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill workload (profiling the decode alone)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--schedule-sweep", action="store_true",
                    help="instead of the benchmark: time one SWA and one global prefill layer at 4K..256K tokens and "
                         "compose the 5:1, 3:1, 1:1 and all-global 32-layer schedules (one JSON line)")
    ap.add_argument("--layers", action="store_true",
                    help="instead of the benchmark: time whole layers from the hidden state (projections on hipBLASLt, "
                         "attention core, o_proj) at 1 x 16384 tokens, d_model 4096 (one JSON line)")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the benchmark: time the training forward and backward of one gated-SWA and one "
                         "global layer at 1 x 16384 tokens (one JSON line)")
    ap.add_argument("--chunked", action="store_true",
                    help="instead of the benchmark: prefill one 262,144-token sequence in 16,384-token chunks through "
                         "the 32-layer schedule against the KV cache (one JSON line)")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="instead of the benchmark: time torch's fp16 matmul (hipBLASLt) on three large square-ish "
                         "GEMMs, the practical MFMA ceiling of this GPU (one JSON line)")
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="also copy a GIB-sized device tensor 3 times (a plain copy kernel of known traffic, for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention core here runs on a single MI355X "
              "(no sharding or collectives); use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import global_attention_gated_amd as zg
    torch.cuda.set_device(0)
    if args.copy_calibration > 0:
        n = int(args.copy_calibration * 2**30) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 2.0, out=dst)      # one elementwise kernel: reads n*4 bytes, writes n*4 bytes
        sync()
        log(f"copy calibration: 3 elementwise copies of {n * 4} bytes (read {n * 4} B + write {n * 4} B each)")
        del src, dst
        torch.cuda.empty_cache()
    if args.gemm_ceiling:
        print(json.dumps({
            "metric": "dense fp16 GEMM TFLOP/s (vendor library), context for the MFMA roofline",
            "unit": "TFLOP/s", "n_gpus": 1, "data": "synthetic", "higher_is_better": True, "dtype": "fp16",
            "config": {"workload": "torch.matmul fp16, 20 timed calls per shape"}, "peak": MFMA_PEAK_TFLOPS,
            "gemms": run_gemm_ceiling(),
        }), flush=True)
        return
    if args.chunked:
        res = run_chunked(zg)
        log(f"chunked: {res['ms_total']:.1f} ms, {res['tokens_per_s']:.0f} tokens/s, global tile kernel "
            f"{res['global_kernel']['tflops']:.0f} TFLOP/s")
        print(json.dumps({
            "metric": "long-context chunked prefill tokens/s + % of MFMA roofline (global layers)",
            "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "data": "synthetic",
            "higher_is_better": True, "dtype": "fp16", "ms_per_step": res["ms_total"],
            "config": {"workload": "one 262,144-token sequence prefilled in 16,384-token chunks, 32-layer schedule "
                                   "(27 gated SWA + 5 global) against the KV cache", "batch": 1, "seq_len": 262144,
                       "chunk": 16384, "layers": N_LAYERS, "global_layers": list(GLOBAL_LAYERS), "q_heads": HQ,
                       "kv_heads": HKV, "head_dim": D, "window": W, "rotary_dims": R, "rope_base": 1e7, "seed": 1005},
            "roofline": res["roofline"], "chunked": res,
        }), flush=True)
        return
    if args.backward:
        res = run_backward(zg, steps=args.steps, warmup=args.warmup)
        print(json.dumps({
            "metric": "training forward + backward time of one attention layer (gradients of q, k, v, gate, norm weights)",
            "unit": "ms", "n_gpus": 1, "data": "synthetic", "higher_is_better": False, "dtype": "bf16",
            "config": {"workload": "one gated-SWA and one global layer, 1 x 16384 tokens", "q_heads": HQ,
                       "kv_heads": HKV, "head_dim": D, "window": W, "rotary_dims": R, "seed": 1008},
            "backward": res,
        }), flush=True)
        return
    if args.layers:
        res = run_layers(zg, steps=args.steps, warmup=args.warmup)
        print(json.dumps({
            "metric": "attention-layer time from the hidden state (q/k/v/g projections + core + o_proj)",
            "unit": "ms", "n_gpus": 1, "data": "synthetic", "higher_is_better": False, "dtype": "bf16",
            "config": {"workload": "one gated-SWA and one global layer, 1 x 16384 tokens", "d_model": D_MODEL,
                       "q_heads": HQ, "kv_heads": HKV, "head_dim": D, "window": W, "rotary_dims": R, "seed": 1007},
            "layers": res,
        }), flush=True)
        return
    if args.schedule_sweep:
        per_layer, sched = run_schedule_sweep(zg)
        for name in SCHEDULES:
            log(f"sweep: {name:10s} " + "  ".join(
                f"{r['seq_len'] // 1024}K {r['attention_ms']:.1f} ms x{r['speedup_vs_all_global']:.2f} "
                f"KV {r['kv_cache_bytes'] / 2**30:.3f} GiB" for r in sched[name]["by_length"]))
        print(json.dumps({
            "metric": "attention time of one 32-layer prefill pass per schedule (sum of measured per-layer times)",
            "unit": "ms", "n_gpus": 1, "data": "synthetic", "higher_is_better": False,
            "config": {"workload": "schedule sweep, batch 1, 4K..256K tokens", "q_heads": HQ, "kv_heads": HKV,
                       "head_dim": D, "window": W, "rotary_dims": R, "rope_base": "1e4 up to 16K, 1e7 above",
                       "seed": 1006, "reps": 3},
            "per_layer_ms": {str(S): v for S, v in per_layer.items()},
            "schedules": sched,
        }), flush=True)
        return
    if args.no_prefill:
        dec = run_decode(zg, args.steps, args.warmup)
        log(f"decode: {dec['ms_per_step']:.3f} ms/step, {dec['tokens_per_s']:.1f} tokens/s, "
            f"split-K kernel {dec['roofline']['achieved']:.0f} GB/s")
        print(json.dumps({"decode": dec}), flush=True)
        return
    log("prefill: setting up 32 layers of 1x16384 inputs")
    pre = run_prefill(zg, args.steps, args.warmup)
    log(f"prefill: {pre['ms_per_step']:.3f} ms/step, {pre['tokens_per_s']:.0f} tokens/s, "
        f"global kernel {pre['kernels']['attn_global']['tflops']:.0f} TFLOP/s, "
        f"SWA kernel {pre['kernels']['attn_swa']['gbs']:.0f} GB/s")
    line = {
        "metric": "attention tokens/s + % of MFMA/HBM roofline (16K SWA prefill; 256K decode)",
        "value": pre["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "precision": "bf16 inputs, outputs and KV cache; fp16 MFMA operands; fp32 accumulation and softmax",
        "data": "synthetic",
        "config": {"workload": "32-layer attention schedule prefill (27 gated SWA + 5 global), 1 x 16384 tokens",
                   "batch": 1, "seq_len": 16384, "layers": N_LAYERS, "global_layers": list(GLOBAL_LAYERS),
                   "q_heads": HQ, "kv_heads": HKV, "head_dim": D, "window": W, "rotary_dims": R, "rope_base": 1e4,
                   "seed": 1003},
        "roofline": pre["roofline"],
        "schedule": {"tflops": pre["schedule_tflops"], "mfma_frac": pre["schedule_mfma_frac"]},
        "kernels": pre["kernels"],
    }
    if not args.no_decode:
        log("decode: allocating and filling the 256K KV cache of 32 sequences")
        dec = run_decode(zg, args.steps, args.warmup)
        log(f"decode: {dec['ms_per_step']:.3f} ms/step, {dec['tokens_per_s']:.1f} tokens/s, "
            f"split-K kernel {dec['roofline']['achieved']:.0f} GB/s")
        line["decode"] = {"metric": "decode tokens/s + % of HBM roofline", "value": dec["tokens_per_s"],
                          "unit": "tokens/s", "ms_per_step": dec["ms_per_step"], "step_gbs": dec["step_gbs"],
                          "step_hbm_frac": dec["step_hbm_frac"], "roofline": dec["roofline"],
                          "kernels": dec["kernels"], "config": dec["config"],
                          "kv_cache_device_bytes": dec["kv_cache_device_bytes"]}
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the fp64 oracle on a sample")
        t0 = time.perf_counter()
        cb = cpu_baseline()
        cb["seconds"] = round(time.perf_counter() - t0, 1)
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
