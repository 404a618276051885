#!/usr/bin/env python3
"""Decode-step benchmark of the TurboQuant compressed-KV hot path on one MI355X.

Workload (default): batched decode, batch 16, 32 query heads / 8 kv-heads (GQA 4), d = 128,
context 131072 per sequence, bf16 K/V drawn Student-t(5) per coordinate with 4 outlier
channels x8, turbo3 (2-bit key codes + 1-bit sign sketch, 3-bit values).  Its packed cache
(1.81 GB) is resident in HBM.  One step = quantize-on-write of the new token's K and V for
every (batch row, kv-head) (16 x 8 + 16 x 8 vectors) into the packed cache, with the query
rotation in the same launch, then decode attention of the 512 (batch row, q-head) pairs over
the full context straight from the codes (tq_decode_step).  The step is captured once in a
HIP graph and replayed.

Prints one JSON line: keys/s (value), the roofline of the dominant kernel (the main
decode-attention kernel: algorithmic bytes per launch over its average duration, timed with
HIP events on its stream), and the oracle's rate on the host cores (cpu_baseline).  Further
workloads (the Llama-3.1-8B decode layer as 32 layers at turbo3 and turbo4, the 70B-shaped
layer, the 1M-context layer) and the uncompressed bf16 comparator go to "extra".
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
HEADLINE = ("c3_batch16_t128k", "turbo3")
# workloads whose 32-layer decode step is timed as well (caches of one layer fit the 256 MB
# Infinity Cache, so 32 distinct layers are cycled)
EXTRA_STEPS = [("c2_llama8b_layer_t32k", "turbo3"), ("c2_llama8b_layer_t32k", "turbo4"),
               ("c2_llama8b_layer_t32k", "k8v4")]
OTHER_WORKLOADS = [("c4_llama70b_layer_b8_t128k", "qjl1"), ("c5_moe_attn_t1m", "turbo3"),
                   ("c5_moe_attn_t1m", "turbo4")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE[0])
    ap.add_argument("--preset", default=HEADLINE[1], choices=["turbo2", "turbo3", "turbo4", "qjl1", "k8v4"])
    ap.add_argument("--layers", type=int, default=0,
                    help="distinct layer caches cycled per step (0: 1 when a layer's cache exceeds 1 GiB, else 32)")
    ap.add_argument("--kernel-launches", type=int, default=30,
                    help="eager attention launches timed one by one for the roofline (at least 20)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall time spent timing the oracle on the host cores (0 disables)")
    ap.add_argument("--other-workloads", type=int, default=1,
                    help="also time the extra workloads and the bf16 comparator (0: headline only)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (calibrates the HBM byte counters) and exit")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attend_kernel.json")
# sources of the attention kernel: the counter figures hold only for the build they were taken on
ATTEND_SOURCES = [os.path.join(ROOT, "kv_cache_vector_tq_amd", "csrc", f)
                  for f in ["tq_attend_kernels.h", "tq_attend.hip"] + [f"tq_attend_k{kb}.hip" for kb in range(9)]]


def attend_sources_sha256() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in ATTEND_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str, preset: str):
    """HBM bytes per launch of the attention kernel from the committed counter summary (FETCH_SIZE
    and WRITE_SIZE, each scaled by the same counter's reading for a copy of known size), or None
    when there is none for this workload or the kernel source changed since it was taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
        digest = attend_sources_sha256()
    except (OSError, ValueError):
        return None
    for e in rec.get("entries", []):
        if e.get("workload") == workload and e.get("preset") == preset and e.get("source_sha256") == digest:
            return float(e["hbm_bytes_per_launch"])
    return None


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


def spread(values) -> dict:
    a = np.asarray(values, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def event_pair():
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    return e0, e1


def run_step(name, preset, dev, layers, steps, warmup, launches, keep_host=False):
    """The decode step of one workload over `layers` distinct layer caches: per layer,
    tq_decode_step (the new token's K and V quantized into slot T-1 with the query rotation in
    the same launch, then attention over the T keys), captured in a HIP graph and replayed.
    Also times the bulk quantize that fills the caches, the attention kernel on its own
    (`launches` eager launches, HIP events on its stream) and the append launch."""
    import torch

    import kv_cache_vector_tq_amd as tq
    import tq_workloads as wl

    w = wl.workload(name)
    B, Hkv, Hq, T = w.B, w.Hkv, w.Hq, w.T
    kb, kq, vb = wl.PRESETS[preset]
    log("drawing inputs", w.name, preset)
    K, V = draw_kv(w, dev)
    Qh = wl.host_tensor(w, wl.TENSOR_Q)
    Q = torch.from_numpy(Qh).to(dev).to(K.dtype)
    cb = tq.tq_build_codebook(kb, kq, vb, seed=0)
    dp = tq.upload_params(cb, dev)
    caches = [tq.KVCache(cb, B, Hkv, T, device=dev, zero=False) for _ in range(layers)]
    bytes_per_key = caches[0].bytes_per_token
    zero = torch.zeros(B, dtype=torch.int32, device=dev)

    # prefill: bulk quantize of the first T-1 tokens into every layer, timed per launch
    qs, qe = event_pair()
    tq.tq_profile_events(quant=(qs, qe))
    bulk_ms = []
    Kp, Vp = K[:, :, : T - 1], V[:, :, : T - 1]
    for rep in range(max(layers, 3)):
        tq.tq_quantize_kv(cb, dp, caches[rep % layers], Kp, Vp, zero)
        torch.cuda.synchronize()
        bulk_ms.append(qs.elapsed_time(qe))
    tq.tq_profile_events()
    n_vec = 2 * B * Hkv * (T - 1)
    bulk_b = bulk_bytes(B, Hkv, T - 1, kb, kq, vb)
    bulk_s = float(np.median(bulk_ms[1:])) * 1e-3
    log(f"bulk quantize: {n_vec} vectors in {bulk_s * 1e6:.1f} us ({bulk_b / bulk_s / 1e9:.0f} GB/s)")

    k_new = [K[:, :, T - 1:T].contiguous() for _ in range(layers)]
    v_new = [V[:, :, T - 1:T].contiguous() for _ in range(layers)]
    del K, V, Kp, Vp
    torch.cuda.empty_cache()
    qs_l = [Q.clone() for _ in range(layers)]
    outs = [torch.empty((B, Hq, 128), dtype=torch.float32, device=dev) for _ in range(layers)]
    start = torch.full((B,), T - 1, dtype=torch.int32, device=dev)
    seq = torch.full((B,), T, dtype=torch.int32, device=dev)
    ws = torch.empty(tq.attend_workspace_bytes(cb, dp, caches[0], Hq, T), dtype=torch.uint8, device=dev)

    def step():
        for l in range(layers):
            tq.tq_decode_step(cb, dp, caches[l], k_new[l], v_new[l], start, qs_l[l], seq, T, out=outs[l],
                              workspace=ws)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t0.elapsed_time(t1) / steps
    log(f"{w.name} {preset}: step {step_ms:.4f} ms ({layers} layer(s)), wall {wall:.3f} s for {steps} steps")
    # single steps, from further replays with an event pair around each (outside the timed region)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        graph.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    one_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    del graph

    # the attention kernel alone: eager launches, HIP events on its own stream around it
    a0, a1 = event_pair()
    tq.tq_profile_events(attend=(a0, a1))
    kern_us = []
    for i in range(launches):
        l = i % layers
        tq.tq_attend_decode(cb, dp, caches[l], qs_l[l], seq, T, out=outs[l], workspace=ws)
        torch.cuda.synchronize()
        kern_us.append(a0.elapsed_time(a1) * 1e3)
    tq.tq_profile_events()
    # the step's append launch (new K and V of every unit plus the query rotation)
    tq.tq_profile_events(quant=(qs, qe))
    app_us = []
    for i in range(launches):
        l = i % layers
        tq.tq_decode_step(cb, dp, caches[l], k_new[l], v_new[l], start, qs_l[l], seq, T, out=outs[l],
                          workspace=ws)
        torch.cuda.synchronize()
        app_us.append(qs.elapsed_time(qe) * 1e3)
    tq.tq_profile_events()
    kern = spread(kern_us)
    bytes_per_launch = B * Hkv * T * bytes_per_key
    achieved = bytes_per_launch / (kern["mean"] * 1e-6) / 1e9
    log(f"attention kernel: mean {kern['mean']:.2f} us (median {kern['median']:.2f}), {achieved:.0f} GB/s; "
        f"append launch median {np.median(app_us):.2f} us")
    keys_per_step = layers * B * Hkv * T
    res = {
        "workload": w.name, "preset": preset, "layers": layers, "bytes_per_key": bytes_per_key,
        "step_ms": step_ms, "keys_per_s": keys_per_step / (step_ms * 1e-3),
        "scores_per_s": keys_per_step * w.G / (step_ms * 1e-3),
        "step_gbs": keys_per_step * bytes_per_key / (step_ms * 1e-3) / 1e9,
        "step_ms_spread": spread(one_ms),
        "attend_kernel": {"us": kern, "bytes_per_launch": bytes_per_launch, "gbs": achieved,
                          "frac": achieved / HBM_PEAK_GBS, "keys_per_s": B * Hkv * T / (kern["mean"] * 1e-6),
                          "scores_per_s": B * Hq * T / (kern["mean"] * 1e-6)},
        "append_launch_us": spread(app_us),
        "append_vectors": 2 * B * Hkv,
        "bulk_quantize": {"vectors_per_launch": n_vec, "us_per_launch": bulk_s * 1e6, "vectors_per_s": n_vec / bulk_s,
                          "gbs": bulk_b / bulk_s / 1e9, "frac": bulk_b / bulk_s / 1e9 / HBM_PEAK_GBS},
    }
    if keep_host:
        # host copies of the first units of layer 0 for the oracle on the host cores
        n_units = min(16, B * Hkv)
        units = [(u // Hkv, u % Hkv) for u in range(n_units)]
        res["_host"] = [{n: (None if t is None else t[b, h].cpu().numpy()) for n, t in caches[0].tensors().items()}
                        for b, h in units]
        res["_units"] = units
        res["_q"] = Qh
    del caches, k_new, v_new, ws, outs, qs_l
    torch.cuda.empty_cache()
    return res


def time_workload(name, preset, dev, launches=20):
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
    e0, e1 = event_pair()
    q_ms = []
    tq.tq_profile_events(quant=(e0, e1))
    for _ in range(3):
        tq.tq_quantize_kv(cb, dp, cache, K, V, zero)
        torch.cuda.synchronize()
        q_ms.append(e0.elapsed_time(e1))
    tq.tq_profile_events()
    del K, V
    seq = torch.full((w.B,), w.T, dtype=torch.int32, device=dev)
    ws = torch.empty(tq.attend_workspace_bytes(cb, dp, cache, w.Hq, w.T), dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device=dev)
    tq.tq_attend_decode(cb, dp, cache, Q, seq, w.T, out=out, workspace=ws)
    torch.cuda.synchronize()
    a_us = []
    tq.tq_profile_events(attend=(e0, e1))
    for _ in range(launches):
        tq.tq_attend_decode(cb, dp, cache, Q, seq, w.T, out=out, workspace=ws)
        torch.cuda.synchronize()
        a_us.append(e0.elapsed_time(e1) * 1e3)
    tq.tq_profile_events()
    a = spread(a_us)
    q_s = float(np.median(q_ms[1:])) * 1e-3
    att_bytes = w.B * w.Hkv * w.T * cache.bytes_per_token
    qb = bulk_bytes(w.B, w.Hkv, w.T, kb, kq, vb)
    n_vec = 2 * w.B * w.Hkv * w.T
    res = {"workload": w.name, "preset": preset,
           "attend": {"us": a, "keys_per_s": w.B * w.Hkv * w.T / (a["mean"] * 1e-6),
                      "gbs": att_bytes / (a["mean"] * 1e-6) / 1e9,
                      "frac": att_bytes / (a["mean"] * 1e-6) / 1e9 / HBM_PEAK_GBS, "bytes": att_bytes},
           "bulk_quantize": {"us": q_s * 1e6, "vectors_per_s": n_vec / q_s, "gbs": qb / q_s / 1e9,
                             "frac": qb / q_s / 1e9 / HBM_PEAK_GBS, "vectors": n_vec}}
    del cache, ws, out
    torch.cuda.empty_cache()
    return res


def time_prefill(name, preset, dev, T_p, reps=3):
    """Prefill of a T_p-token prompt into one layer's packed cache: the bulk quantize-on-write of
    its keys and values, then causal attention of its T_p queries (all q-heads) over the packed
    cache (tq_attend_prefill), each timed with HIP events on its stream."""
    import torch

    import kv_cache_vector_tq_amd as tq
    import tq_workloads as wl

    w = wl.workload(name)
    kb, kq, vb = wl.PRESETS[preset]
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.cfg_seed)
    K = torch.randn((w.B, w.Hkv, T_p, 128), generator=gen, device=dev).to(torch.bfloat16)
    V = torch.randn((w.B, w.Hkv, T_p, 128), generator=gen, device=dev).to(torch.bfloat16)
    Q = torch.randn((w.B, w.Hq, T_p, 128), generator=gen, device=dev).to(torch.bfloat16)
    cb = tq.tq_build_codebook(kb, kq, vb, seed=0)
    dp = tq.upload_params(cb, dev)
    cache = tq.KVCache(cb, w.B, w.Hkv, T_p, device=dev, zero=False)
    zero = torch.zeros(w.B, dtype=torch.int32, device=dev)
    out = torch.empty((w.B, w.Hq, T_p, 128), dtype=torch.float32, device=dev)
    e0, e1 = event_pair()
    q_us, a_us = [], []
    for _ in range(reps):
        tq.tq_profile_events(quant=(e0, e1))
        tq.tq_quantize_kv(cb, dp, cache, K, V, zero)
        torch.cuda.synchronize()
        q_us.append(e0.elapsed_time(e1) * 1e3)
        tq.tq_profile_events(attend=(e0, e1))
        tq.tq_attend_prefill(cb, dp, cache, Q, zero, T_p, out=out)
        torch.cuda.synchronize()
        a_us.append(e0.elapsed_time(e1) * 1e3)
    tq.tq_profile_events()
    qs, as_ = float(np.median(q_us)), float(np.median(a_us))
    pairs = w.B * w.Hq * T_p * (T_p + 1) / 2  # (query, visible key) pairs over all q-heads
    res = {"workload": f"{w.name} prompt of {T_p} tokens", "preset": preset, "prompt_tokens": T_p,
           "bulk_quantize_us": qs, "prefill_attention_us": as_, "prompt_tokens_per_s": w.B * T_p / ((qs + as_) * 1e-6),
           "scores_per_s": pairs / (as_ * 1e-6),
           "bulk_quantize_gbs": bulk_bytes(w.B, w.Hkv, T_p, kb, kq, vb) / (qs * 1e-6) / 1e9}
    del K, V, Q, cache, out
    torch.cuda.empty_cache()
    return res


def read_ceiling(dev, mib=4096, grids=(1024, 2048, 4096, 8192), reps=5):
    """The box's streaming read rate: this library's read probe (16-byte loads, one launch over a
    4 GiB buffer, well beyond the 256 MB Infinity Cache) at several grid sizes; the best median
    over `reps` launches per grid."""
    import torch

    import kv_cache_vector_tq_amd as tq

    buf = torch.zeros(mib << 20, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    best, per_grid = 0.0, {}
    for g in grids:
        tq.tq_read_probe(buf, g, sink)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            tq.tq_read_probe(buf, g, sink)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        gbs = buf.numel() / float(np.median(ts)) / 1e9
        per_grid[str(g)] = gbs
        best = max(best, gbs)
    del buf
    torch.cuda.empty_cache()
    return best, per_grid


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

    Vts = [tq.bf16_value_chunks(v) for v in Vs]
    ws = torch.empty(tq.bf16_attend_workspace_bytes(B, Hkv, T, Hq, T), dtype=torch.uint8, device=dev)
    hip_us = timed(lambda: [tq.tq_bf16_attend_decode(Ks[l], Vts[l], q, seq, T, out=out, workspace=ws)
                            for l in range(layers)])
    del Vts
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


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1 (no multi-GPU path "
                                   "is built: the kernels run on one GPU's share of the work)",
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
    kb, kq, vb = wl.PRESETS[args.preset]
    per_layer = w.B * w.Hkv * w.T * tq.tq_cache_layout(kb, kq, vb, 1, 1, 64)["bytes_per_token"]
    layers = args.layers or (1 if per_layer > (1 << 30) else 32)
    launches = max(20, args.kernel_launches)

    log("read probe")
    read_gbs, read_grid = read_ceiling(dev)
    log(f"stream read ceiling {read_gbs:.0f} GB/s {read_grid}")

    head = run_step(w.name, args.preset, dev, layers, args.steps, args.warmup, launches,
                    keep_host=args.cpu_seconds > 0)
    host = (head.pop("_host", None), head.pop("_units", None), head.pop("_q", None))

    steps_extra, others, comparator, prefill = [], [], None, []
    if args.other_workloads:
        for T_p in (4096, 32768):
            log("prefill", T_p)
            prefill.append(time_prefill("c2_llama8b_layer_t32k", "turbo3", dev, T_p))
            log(json.dumps(prefill[-1]))
        for name, preset in EXTRA_STEPS:
            if (name, preset) == (w.name, args.preset):
                continue
            steps_extra.append(run_step(name, preset, dev, 32, args.steps, args.warmup, 2 * 32))
            log(json.dumps(steps_extra[-1]))
        c2 = wl.workload("c2_llama8b_layer_t32k")
        bf16_us, torch_us = bf16_comparator(c2, 32, dev)
        bf16_bytes = 2 * c2.B * c2.Hkv * c2.T * 128 * 2
        c2_call = next((s for s in steps_extra if s["preset"] == "turbo3"), None)
        comparator = {"kind": "uncompressed bf16 decode attention at the Llama-3.1-8B layer shape (32 distinct "
                              "layers): tq_bf16_attend_decode (this library's baseline kernel) and plain PyTorch "
                              "(bmm, fp32 softmax, bmm)",
                      "us_per_layer": bf16_us, "keys_per_s": c2.B * c2.Hkv * c2.T / (bf16_us * 1e-6),
                      "gbs": bf16_bytes / (bf16_us * 1e-6) / 1e9, "torch_us_per_layer": torch_us}
        if c2_call is not None:
            per_layer_us = c2_call["step_ms"] * 1e3 / c2_call["layers"]
            comparator["compressed_step_us_per_layer"] = per_layer_us
            comparator["speedup_of_compressed_step"] = bf16_us / per_layer_us
        log(json.dumps(comparator))
        for name, preset in OTHER_WORKLOADS:
            log("timing", name, preset)
            others.append(time_workload(name, preset, dev))
            log(json.dumps(others[-1]))

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, args.preset, *host, args.cpu_seconds)

    ka = head["attend_kernel"]
    line = {
        "metric": "compressed-KV decode attention keys/s + achieved HBM GB/s (% of peak) at 3/4 bit",
        "value": head["keys_per_s"],
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA operands (query as an f16 hi+lo pair), fp32 accumulation; bf16 MFMA rotation",
        "data": "synthetic",
        "config": {"workload": w.name, "preset": args.preset, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": 128, "context": w.T, "layers": layers, "bytes_per_key": head["bytes_per_key"],
                   "step": f"tq_decode_step: quantize-on-write of {w.B}x{w.Hkv} new K and V vectors (query rotation "
                           f"in the same launch), then decode attention of {w.B * w.Hq} (batch row, q-head) pairs "
                           f"over {w.T} keys"},
        "roofline": {"bound": "hbm", "achieved": ka["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ka["frac"], "traffic": measured_traffic(w.name, args.preset),
                     "kernel": "attend_kernel (main decode attention)", "bytes_per_launch": ka["bytes_per_launch"],
                     "avg_launch_us": ka["us"]["mean"], "launches": ka["us"]["n"]},
        "cpu_baseline": cpu,
        "extra": {
            "headline": head,
            "measured_read_gbs": read_gbs,
            "read_probe_gbs_by_grid": read_grid,
            "attend_frac_of_measured_read": ka["gbs"] / read_gbs,
            "steps": steps_extra,
            "workloads": others,
            "prefill": prefill,
            "bf16_comparator": comparator,
            "targets": {"attend_frac": 0.70, "quantize_frac": 0.60},
        },
    }
    print(json.dumps(line), flush=True)


def _oracle_unit_worker(job):
    """One host core: the oracle (fp64 NumPy, one BLAS thread) decoding one (batch row, kv-head)
    unit from its packed cache (unpack + attention of its G q-heads over T keys) until `seconds`
    have passed, then quantizing 2048 keys + 2048 values of the same slice for seconds / 4."""
    preset, unit_cache, q, T, workload, b, h, seconds = job
    from threadpoolctl import threadpool_limits

    import tq_workloads as wl
    from oracle.pipeline import Oracle

    with threadpool_limits(limits=1):
        orc = Oracle(*wl.PRESETS[preset], seed=0)
        reps, t0 = 0, time.perf_counter()
        while True:
            k = orc.unpack_keys(unit_cache["k_codes"], unit_cache["k_signs"], unit_cache["k_norm"],
                                unit_cache["k_rnorm"], T)
            v = orc.unpack_values(unit_cache["v_codes"], unit_cache["v_norm"], T)
            orc.attend(q, k, v, T=T)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        w = wl.workload(workload)
        xk = wl.host_slice(w, b, h, wl.TENSOR_K, n=2048).astype(np.float64)
        xv = wl.host_slice(w, b, h, wl.TENSOR_V, n=2048).astype(np.float64)
        qreps, q0 = 0, time.perf_counter()
        while True:
            orc.quantize_keys(xk)
            orc.quantize_values(xv)
            qreps += 1
            qel = time.perf_counter() - q0
            if qel >= seconds / 4:
                break
    return reps, el, qreps, qel


def cpu_baseline(w, preset, host_units, units, Qh, seconds):
    """The oracle on the host cores: one worker process per core (at most 16, the GPU's share of
    the box), each single-threaded, each decoding a different (batch row, kv-head) unit of the
    workload from the GPU-written packed cache at full context, repeated for about `seconds`.
    keys/s = keys attended by all workers / wall time."""
    import concurrent.futures
    import multiprocessing

    try:
        n_cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n_cores = os.cpu_count() or 1
    workers = max(1, min(16, n_cores, len(host_units)))
    jobs = []
    for i in range(workers):
        b, h = units[i]
        jobs.append((preset, host_units[i], Qh[b, h * w.G:(h + 1) * w.G].astype(np.float64), w.T, w.name, b, h,
                     seconds))
    ctx = multiprocessing.get_context("spawn")
    t0 = time.perf_counter()
    with concurrent.futures.ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        res = list(ex.map(_oracle_unit_worker, jobs))
    wall = time.perf_counter() - t0
    keys = sum(r[0] for r in res) * w.T
    att_rate = sum(r[0] * w.T / r[1] for r in res)
    q_rate = sum(r[2] * 4096 / r[3] for r in res)
    return {"value": att_rate, "unit": "keys/s", "cores": workers, "kind": "oracle",
            "sample": f"{workers} worker processes (one BLAS thread each), each decoding a different (batch row, "
                      f"kv-head) unit of {w.name} {preset} from the GPU-written cache: unpack + attention of "
                      f"{w.G} q-heads over {w.T} keys, fp64 NumPy; {sum(r[0] for r in res)} unit passes, "
                      f"{keys} keys in {wall:.1f} s of wall time (value = sum of per-worker rates)",
            "quantize_vectors_per_s": q_rate,
            "quantize_sample": "per worker: 2048 keys + 2048 values of its unit, repeated for "
                               f"{seconds / 4:.1f} s (sum of per-worker rates)",
            "cpu_model": host_cpu_model(), "host_cpus": n_cores}


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
