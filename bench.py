#!/usr/bin/env python3
"""Decode-step benchmark of the TurboQuant compressed-KV hot path on one MI355X.

Workload: a Llama-3.1-8B-shaped decode layer (batch 1, 32 q-heads / 8 kv-heads, d = 128,
context 32768, bf16 K/V ~ N(0,1) x per-channel LogNormal(0, 0.5) scales), stacked as 32
layers with distinct caches so that the packed caches (32 x 28.3 MB at turbo3) do not
fit the 256 MB Infinity Cache.  One step = for every layer: quantize-on-write of the new
token's K and V (8 + 8 vectors) into the packed cache, then decode attention of the 32
q-heads over the 32768-key context straight from the codes.  The step is captured once
in a HIP graph and replayed.

Prints one JSON line: keys/s (value), the roofline of the dominant kernel (the main
decode-attention kernel: algorithmic bytes per launch over its average duration, timed
with HIP events on its stream), and the oracle's rate on the host cores (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--preset", default="turbo3", choices=["turbo3", "turbo4", "qjl1"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall time spent timing the oracle on the host (0 disables)")
    ap.add_argument("--kernel-reps", type=int, default=4, help="eager passes over the layers for kernel timing")
    ap.add_argument("--workload", default="c2_llama8b_layer_t32k",
                    help="workload name (default: the Llama-3.1-8B decode layer); others are for exploration")
    ap.add_argument("--other-workloads", type=int, default=1,
                    help="also time the attention kernel and bulk quantize on the other HBM-sized workloads (0: off)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (calibrates the HBM byte counters) and exit")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attend_kernel.json")
# sources of the attention kernel: the counter figures hold only for the build they were taken on
ATTEND_SOURCES = [os.path.join(ROOT, "kv_cache_vector_tq_amd", "csrc", f)
                  for f in ["tq_attend_kernels.h", "tq_attend.hip"] + [f"tq_attend_k{kb}.hip" for kb in range(5)]]


def measured_traffic(workload: str, preset: str):
    """HBM bytes per launch of the attention kernel from the committed counter summary (FETCH_SIZE
    and WRITE_SIZE, each scaled by the same counter's reading for a copy of known size), or None
    when there is none for this workload or the kernel source changed since it was taken."""
    import hashlib

    try:
        rec = json.load(open(TRAFFIC_FILE))
        h = hashlib.sha256()
        for f in ATTEND_SOURCES:
            h.update(open(f, "rb").read())
        digest = h.hexdigest()
    except (OSError, ValueError):
        return None
    for e in rec.get("entries", []):
        if e.get("workload") == workload and e.get("preset") == preset and e.get("source_sha256") == digest:
            return float(e["hbm_bytes_per_launch"])
    return None


OTHER_WORKLOADS = [("c3_batch16_t128k", "turbo3"), ("c4_llama70b_layer_b8_t128k", "qjl1"),
                   ("c5_moe_attn_t1m", "turbo3"), ("c5_moe_attn_t1m", "turbo4")]


def draw_kv(w, dev):
    """K and V of a workload on the device (bf16/fp32), drawn from the seeded generators."""
    import torch

    import tq_workloads as wl

    in_dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    if w.B * w.Hkv * w.T <= (1 << 19):
        K = torch.from_numpy(wl.host_tensor(w, wl.TENSOR_K)).to(dev).to(in_dtype)
        V = torch.from_numpy(wl.host_tensor(w, wl.TENSOR_V)).to(dev).to(in_dtype)
    else:  # large contexts are drawn on the device, one (b, kv-head) slice at a time
        K = torch.empty((w.B, w.Hkv, w.T, 128), dtype=in_dtype, device=dev)
        V = torch.empty((w.B, w.Hkv, w.T, 128), dtype=in_dtype, device=dev)
        for bb in range(w.B):
            for hh in range(w.Hkv):
                wl.device_slice(w, bb, hh, wl.TENSOR_K, out=K[bb, hh])
                wl.device_slice(w, bb, hh, wl.TENSOR_V, out=V[bb, hh])
    return K, V


def bulk_bytes(B, Hkv, n, kb, kq, vb):
    k_out = 16 * kb + (16 if kq else 0) + 4 + (4 if (kq and kb) else 0)
    v_out = 16 * vb + 4
    return B * Hkv * n * (256 + k_out) + B * Hkv * n * (256 + v_out)


def time_workload(name, preset, dev, reps=5):
    """Attention kernel (HIP events on its stream) and bulk quantize of the full context for one
    workload: one cache, inputs resident in HBM."""
    import torch

    import kv_cache_vector_tq_amd as tq
    import tq_workloads as wl

    w = wl.workload(name)
    kb, kq, vb = wl.PRESETS[preset]
    K, V = draw_kv(w, dev)
    Q = torch.from_numpy(wl.host_tensor(w, wl.TENSOR_Q)).to(dev).to(K.dtype)
    cb = tq.tq_build_codebook(kb, kq, vb, seed=0)
    dp = tq.upload_params(cb, dev)
    cache = tq.KVCache(cb, w.B, w.Hkv, w.T, device=dev, zero=False)
    zero = torch.zeros(w.B, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    q_ms = []
    tq.tq_profile_events(quant=(e0, e1))
    for _ in range(3):
        tq.tq_quantize_kv(cb, dp, cache, K, V, zero)
        torch.cuda.synchronize()
        q_ms.append(e0.elapsed_time(e1))
    tq.tq_profile_events()
    del K, V
    seq = torch.full((w.B,), w.T, dtype=torch.int32, device=dev)
    ws = torch.zeros(tq.attend_workspace_bytes(cb, dp, cache, w.Hq, w.T), dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device=dev)
    tq.tq_attend_decode(cb, dp, cache, Q, seq, w.T, out=out, workspace=ws)
    torch.cuda.synchronize()
    a_ms = []
    tq.tq_profile_events(attend=(e0, e1))
    for _ in range(reps):
        tq.tq_attend_decode(cb, dp, cache, Q, seq, w.T, out=out, workspace=ws)
        torch.cuda.synchronize()
        a_ms.append(e0.elapsed_time(e1))
    tq.tq_profile_events()
    a_s = float(np.median(a_ms)) * 1e-3
    q_s = float(np.median(q_ms[1:])) * 1e-3
    att_bytes = w.B * w.Hkv * w.T * cache.bytes_per_token
    qb = bulk_bytes(w.B, w.Hkv, w.T, kb, kq, vb)
    n_vec = 2 * w.B * w.Hkv * w.T
    res = {"workload": w.name, "preset": preset,
           "attend": {"us": a_s * 1e6, "keys_per_s": w.B * w.Hkv * w.T / a_s, "gbs": att_bytes / a_s / 1e9,
                      "frac": att_bytes / a_s / 1e9 / HBM_PEAK_GBS, "bytes": att_bytes},
           "bulk_quantize": {"us": q_s * 1e6, "vectors_per_s": n_vec / q_s, "gbs": qb / q_s / 1e9,
                             "frac": qb / q_s / 1e9 / HBM_PEAK_GBS, "vectors": n_vec}}
    del cache, ws, out
    torch.cuda.empty_cache()
    return res


def stream_read_gbs(dev, mib=2048):
    """Read bandwidth of the box: row sums over a 2 GiB fp32 buffer (a streaming read that
    writes almost nothing), 5 passes timed with events."""
    import torch

    x = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    xv = x.view(4096, -1)
    xv.sum(dim=1)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(5):
        xv.sum(dim=1)
    t1.record()
    torch.cuda.synchronize()
    gbs = 5 * x.numel() * 4 / (t0.elapsed_time(t1) * 1e-3) / 1e9
    del x
    torch.cuda.empty_cache()
    return gbs


def bf16_comparator(w, layers, dev, reps=3):
    """Uncompressed bf16 decode attention at the same shape, `layers` distinct K/V caches, timed
    back to back: (a) this library's bf16 baseline kernel (tq_bf16_attend_decode, V stored
    transposed per 32-key chunk), (b) plain PyTorch (bmm with contiguous operands, fp32
    softmax, bmm).  Returns us per layer of each."""
    import torch

    import kv_cache_vector_tq_amd as tq

    B, Hkv, Hq, G, T = w.B, w.Hkv, w.Hq, w.G, w.T
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    Ks = [torch.randn((B, Hkv, T, 128), generator=gen, device=dev).to(torch.bfloat16) for _ in range(layers)]
    Vs = [torch.randn((B, Hkv, T, 128), generator=gen, device=dev).to(torch.bfloat16) for _ in range(layers)]
    q = torch.randn((B, Hq, 128), generator=gen, device=dev).to(torch.bfloat16)
    seq = torch.full((B,), T, dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / (reps * layers)

    # (a) baseline kernel
    Vts = [tq.bf16_value_chunks(v) for v in Vs]
    ws = torch.empty(tq.bf16_attend_workspace_bytes(B, Hkv, T, Hq, T), dtype=torch.uint8, device=dev)
    hip_us = timed(lambda: [tq.tq_bf16_attend_decode(Ks[l], Vts[l], q, seq, T, out=out, workspace=ws)
                            for l in range(layers)])
    del Vts
    # (b) plain PyTorch, one bmm per kv-head group
    qT = q.view(B * Hkv, G, 128).transpose(1, 2).contiguous()  # [B*Hkv, 128, G]
    scale = 1.0 / math.sqrt(128)

    def layer(K, V):
        sc = torch.bmm(K.view(B * Hkv, T, 128), qT).float() * scale  # [B*Hkv, T, G]
        p = torch.softmax(sc, dim=1).to(torch.bfloat16).transpose(1, 2).contiguous()  # [B*Hkv, G, T]
        return torch.bmm(p, V.view(B * Hkv, T, 128))  # [B*Hkv, G, 128]

    torch_us = timed(lambda: [layer(K, V) for K, V in zip(Ks, Vs)])
    del Ks, Vs
    torch.cuda.empty_cache()
    return hip_us, torch_us


def copy_probe(mib: int):
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "copies": 5}), flush=True)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import torch

    import kv_cache_vector_tq_amd as tq
    import tq_workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.workload(args.workload)
    B, Hkv, Hq, T, G = w.B, w.Hkv, w.Hq, w.T, w.G
    L = args.layers
    kb, kq, vb = wl.PRESETS[args.preset]

    # ---- inputs (seeded, synthetic) -------------------------------------------------------------
    log("drawing inputs", w.name)
    K, V = draw_kv(w, dev)
    Qh = wl.host_tensor(w, wl.TENSOR_Q)
    Q = torch.from_numpy(Qh).to(dev).to(K.dtype)

    cb = tq.tq_build_codebook(kb, kq, vb, seed=0)
    dp = tq.upload_params(cb, dev)
    caches = [tq.KVCache(cb, B, Hkv, T, device=dev, zero=False) for _ in range(L)]
    bytes_per_key = caches[0].bytes_per_token
    zero = torch.zeros(B, dtype=torch.int32, device=dev)

    # ---- prefill: bulk quantize of T-1 tokens into every layer (timed per launch) ---------------
    qs, qe = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qs.record()
    qe.record()
    torch.cuda.synchronize()
    tq.tq_profile_events(quant=(qs, qe))
    bulk_ms = []
    Kp, Vp = K[:, :, : T - 1], V[:, :, : T - 1]
    for l in range(L):
        tq.tq_quantize_kv(cb, dp, caches[l], Kp, Vp, zero)
        torch.cuda.synchronize()
        bulk_ms.append(qs.elapsed_time(qe))
    tq.tq_profile_events()
    n_vec = 2 * B * Hkv * (T - 1)
    bulk_b = bulk_bytes(B, Hkv, T - 1, kb, kq, vb)
    bulk_s = float(np.median(bulk_ms[1:] if L > 1 else bulk_ms)) * 1e-3
    log(f"bulk quantize: {n_vec} vectors in {bulk_s * 1e6:.1f} us")

    # ---- one decode step over all layers ----------------------------------------------------------
    k_new = [K[:, :, T - 1:T].contiguous() for _ in range(L)]
    v_new = [V[:, :, T - 1:T].contiguous() for _ in range(L)]
    qs_l = [Q.clone() for _ in range(L)]
    outs = [torch.empty((B, Hq, 128), dtype=torch.float32, device=dev) for _ in range(L)]
    start = torch.full((B,), T - 1, dtype=torch.int32, device=dev)
    seq = torch.full((B,), T, dtype=torch.int32, device=dev)
    ws = torch.zeros(tq.attend_workspace_bytes(cb, dp, caches[0], Hq, T), dtype=torch.uint8, device=dev)

    # per layer: the new token's quantize-on-write, then attention (tq_decode_step: the query
    # rotation rides in the quantize launch, so two launches per layer)
    def step():
        for l in range(L):
            tq.tq_decode_step(cb, dp, caches[l], k_new[l], v_new[l], start, qs_l[l], seq, T, out=outs[l],
                              workspace=ws)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t0.elapsed_time(t1) / args.steps
    keys_per_step = L * B * Hkv * T
    value = keys_per_step / (step_ms * 1e-3)
    log(f"step {step_ms:.3f} ms ({L} layers), wall {wall:.3f} s for {args.steps} steps")
    # spread of single steps, from further replays with an event pair around each (outside the
    # timed region above, which `value` comes from)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record()
    for i in range(args.steps):
        graph.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    one_ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    step_spread = {"median": float(np.median(one_ms)), "p10": float(np.percentile(one_ms, 10)),
                   "p90": float(np.percentile(one_ms, 90)), "steps": args.steps}

    # ---- dominant kernel: main attention kernel, HIP events on its stream ------------------------
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    a1.record()
    torch.cuda.synchronize()
    tq.tq_profile_events(attend=(a0, a1))
    kern_ms = []
    for _ in range(args.kernel_reps):
        for l in range(L):
            tq.tq_attend_decode(cb, dp, caches[l], qs_l[l], seq, T, out=outs[l], workspace=ws)
            torch.cuda.synchronize()
            kern_ms.append(a0.elapsed_time(a1))
    tq.tq_profile_events()
    kern_s = float(np.mean(kern_ms)) * 1e-3
    kern_us = np.array(kern_ms) * 1e3
    kern_spread = {"median": float(np.median(kern_us)), "p10": float(np.percentile(kern_us, 10)),
                   "p90": float(np.percentile(kern_us, 90)), "launches": len(kern_ms)}
    bytes_per_launch = B * Hkv * T * bytes_per_key
    achieved = bytes_per_launch / kern_s / 1e9
    log(f"attention kernel: {kern_s * 1e6:.2f} us per launch, {achieved:.0f} GB/s")

    # whole attention call (query prologue + main kernel) per layer, back to back over the layers
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(args.kernel_reps):
        for l in range(L):
            tq.tq_attend_decode(cb, dp, caches[l], qs_l[l], seq, T, out=outs[l], workspace=ws)
    c1.record()
    torch.cuda.synchronize()
    call_us = c0.elapsed_time(c1) * 1e3 / (args.kernel_reps * L)
    log(f"attention call (prologue + main): {call_us:.2f} us per layer")

    # host copy of one (batch row, kv-head) of layer 0 for the oracle on the host cores
    host = {n: (None if t is None else t[0, 0].cpu().numpy()) for n, t in caches[0].tensors().items()}

    # ---- the other HBM-sized workloads (one cache each; the step's caches are freed first) -------
    others = []
    comparator = None
    if args.other_workloads:
        del caches, k_new, v_new, K, V, ws, outs, qs_l, graph
        torch.cuda.empty_cache()
        bf16_us, torch_us = bf16_comparator(w, L, dev)
        bf16_bytes = 2 * B * Hkv * T * 128 * 2
        comparator = {"kind": "uncompressed bf16 decode attention, same shape: tq_bf16_attend_decode (this "
                              "library's baseline kernel) and plain PyTorch (bmm, fp32 softmax, bmm)",
                      "us_per_layer": bf16_us, "keys_per_s": B * Hkv * T / (bf16_us * 1e-6),
                      "gbs": bf16_bytes / (bf16_us * 1e-6) / 1e9,
                      "torch_us_per_layer": torch_us,
                      "compressed_call_us_per_layer": call_us,
                      "speedup_of_compressed_call": bf16_us / call_us}
        log(json.dumps(comparator))
        for name, preset in OTHER_WORKLOADS:
            log("timing", name, preset)
            others.append(time_workload(name, preset, dev))
            log(json.dumps(others[-1]))
    read_gbs = stream_read_gbs(dev)
    log(f"stream read ceiling {read_gbs:.0f} GB/s")

    # ---- oracle on the host cores ----------------------------------------------------------------
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, host, Qh, args.preset, args.cpu_seconds)

    line = {
        "metric": "compressed-KV decode attention keys/s + achieved HBM GB/s (% of peak) at 3/4 bit",
        "value": value,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "preset": args.preset, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": 128, "context": T, "layers": L, "bytes_per_key": bytes_per_key,
                   "step": "per layer: quantize-on-write of 1 new token (K+V) then decode attention (tq_decode_step)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(w.name, args.preset),
                     "kernel": "attend_kernel (main decode attention)", "bytes_per_launch": bytes_per_launch,
                     "avg_launch_us": kern_s * 1e6},
        "cpu_baseline": cpu,
        "extra": {
            "attend_frac_of_measured_read": achieved / read_gbs,
            "measured_read_gbs": read_gbs,
            "workloads": others,
            "attend_call_us_per_layer": call_us,
            "bf16_comparator": comparator,
            "step_gbs": keys_per_step * bytes_per_key / (step_ms * 1e-3) / 1e9,
            "step_ms_spread": step_spread,
            "scores_per_s": keys_per_step * G / (step_ms * 1e-3),
            "attend_launch_us_spread": kern_spread,
            "attend_kernel_scores_per_s": B * Hq * T / kern_s,
            "bulk_quantize": {"vectors_per_launch": n_vec, "us_per_launch": bulk_s * 1e6,
                              "vectors_per_s": n_vec / bulk_s, "gbs": bulk_b / bulk_s / 1e9,
                              "frac": bulk_b / bulk_s / 1e9 / HBM_PEAK_GBS},
        },
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(w, host, Qh, preset, seconds):
    """The oracle (fp64 NumPy) decoding one (batch row, kv-head) of one layer from its packed cache:
    unpack the codes, then attention of the G q-heads over the full context.  Repeated for
    about `seconds`; reported as keys/s (keys attended per second)."""
    import tq_workloads as wl
    from oracle.pipeline import Oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    orc = Oracle(*wl.PRESETS[preset], seed=0)
    T, G = w.T, w.G
    q = Qh[0, :G].astype(np.float64)
    reps = 0
    t0 = time.perf_counter()
    while True:
        k = orc.unpack_keys(host["k_codes"], host["k_signs"], host["k_norm"], host["k_rnorm"], T)
        v = orc.unpack_values(host["v_codes"], host["v_norm"], T)
        orc.attend(q, k, v, T=T)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    # quantize-on-write: the oracle quantizing the first 2048 keys and values of the same slice
    xk = wl.host_slice(w, 0, 0, wl.TENSOR_K, n=2048).astype(np.float64)
    xv = wl.host_slice(w, 0, 0, wl.TENSOR_V, n=2048).astype(np.float64)
    qreps = 0
    q0 = time.perf_counter()
    while True:
        orc.quantize_keys(xk)
        orc.quantize_values(xv)
        qreps += 1
        qel = time.perf_counter() - q0
        if qel >= seconds / 4:
            break
    return {"value": reps * T / el, "unit": "keys/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} decode passes of one (batch row, kv-head) of one layer: unpack + attention of "
                      f"{G} q-heads over {T} keys, fp64 NumPy ({el:.1f} s)",
            "quantize_vectors_per_s": qreps * 4096 / qel,
            "quantize_sample": f"{qreps} x (2048 keys + 2048 values) of the same slice ({qel:.1f} s)",
            "cpu_model": host_cpu_model(), "host_cpus": os.cpu_count()}


def host_cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
