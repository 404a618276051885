"""GPU parity of the HIP path against the oracle (small and mid-size workloads, edge cases).

Every call goes through libtq's C ABI (kv_cache_vector_tq_amd binds it with ctypes).
"""
import contextlib
import math
import os
import sys

import numpy as np
import pytest

import tq_workloads as wl
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU machines deselect these tests
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_vector_tq_amd as tq  # noqa: E402


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


@contextlib.contextmanager
def attention_tables(repl):
    """TQ_ATTN_REPL for the calls inside: "1" forces the attention kernel instance with decode
    tables replicated per lane slot (chosen by itself only for long streams), "auto" leaves the
    choice to the library."""
    old = os.environ.get("TQ_ATTN_REPL")
    if repl == "auto":
        os.environ.pop("TQ_ATTN_REPL", None)
    else:
        os.environ["TQ_ATTN_REPL"] = repl
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("TQ_ATTN_REPL", None)
        else:
            os.environ["TQ_ATTN_REPL"] = old


def _setup(preset, B, Hkv, T_cap, seed=0, zero=True, rotation="haar"):
    cb = tq.tq_build_codebook(*(wl.PRESETS[preset] if isinstance(preset, str) else preset), seed=seed,
                              rotation=rotation)
    dp = tq.upload_params(cb)
    cache = tq.KVCache(cb, B, Hkv, T_cap, zero=zero)
    return cb, dp, cache


def _run_workload_full(w, preset):
    """Quantize the whole workload and attend once; return everything for the comparison."""
    K = wl.host_tensor(w, wl.TENSOR_K)
    V = wl.host_tensor(w, wl.TENSOR_V)
    Q = wl.host_tensor(w, wl.TENSOR_Q)
    cb, dp, cache = _setup(preset, w.B, w.Hkv, wl.round_up(w.T, 64))
    say(w.name, preset, "quantize", K.shape)
    start = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    tq.tq_quantize_kv(cb, dp, cache, H.to_device(K, w.dtype), H.to_device(V, w.dtype), start)
    seq = torch.full((w.B,), w.T, dtype=torch.int32, device="cuda")
    scores = torch.zeros((w.B, w.Hq, cache.T_cap), dtype=torch.float32, device="cuda")
    say(w.name, preset, "attend")
    out = tq.tq_attend_decode(cb, dp, cache, H.to_device(Q, w.dtype), seq, w.T, scores_out=scores)
    torch.cuda.synchronize()
    say(w.name, preset, "device done")
    q_used = Q if w.dtype == "f32" else wl.round_to_bf16(Q)
    return K, V, q_used, H.cache_host(cache), out.cpu().numpy(), scores.cpu().numpy()


@pytest.mark.parametrize("wname,preset", [("c1_single_head_t4096", "turbo3"),
                                          ("c2_llama8b_layer_t32k", "turbo3"),
                                          ("c2_llama8b_layer_t32k", "turbo4"),
                                          ("c2_llama8b_layer_t32k", "k8v4")])
def test_workload_parity(wname, preset):
    w = wl.workload(wname)
    K, V, Q, hc, out, scores = _run_workload_full(w, preset)
    orc = H.make_oracle(preset)
    stats, errs = {}, []
    for b in range(w.B):
        for h in range(w.Hkv):
            kg = H.unpack_keys(orc, hc, b, h, w.T)
            vg = H.unpack_values(orc, hc, b, h, w.T)
            H.compare_keys(orc, K[b, h], kg, stats)
            H.compare_values(orc, V[b, h], vg, stats)
            hs = slice(h * w.G, (h + 1) * w.G)
            errs.append(H.compare_attention(orc, Q[b, hs], kg, vg, w.T, out[b, hs], scores[b, hs]))
    H.finish_stats(stats)
    say(wname, preset, "codes", stats, "max rel err", max(e["out"] for e in errs), max(e["score_vs_rowmax"] for e in errs))


@pytest.mark.parametrize("wname,preset", [("c3_batch16_t128k", "turbo3"), ("c4_llama70b_layer_b8_t128k", "qjl1"),
                                          ("c5_moe_attn_t1m", "turbo3"), ("c5_moe_attn_t1m", "turbo4")])
def test_full_size_sampled(wname, preset):
    """The large workloads at full size, in the calls and launch shapes the benchmark times:
    the whole context quantized by one call, one attention call over every (batch row,
    kv-head) unit, inputs drawn on the device by the seeded workload generator.  The oracle
    checks the first and the last unit: codes, signs and norms of a token sample (the first
    and last 64-token blocks plus 16384 random tokens), and every q-head's output over the
    full context (decoded from the GPU-written cache)."""
    w = wl.workload(wname)
    T = w.T
    cb, dp, cache = _setup(preset, w.B, w.Hkv, T, zero=False)
    K = torch.empty((w.B, w.Hkv, T, 128), dtype=torch.bfloat16, device="cuda")
    V = torch.empty_like(K)
    for b in range(w.B):
        for h in range(w.Hkv):
            wl.device_slice(w, b, h, wl.TENSOR_K, out=K[b, h])
            wl.device_slice(w, b, h, wl.TENSOR_V, out=V[b, h])
    g = torch.Generator(device="cuda")
    g.manual_seed(w.cfg_seed)
    Q = torch.randn((w.B, w.Hq, 128), generator=g, device="cuda").to(torch.bfloat16)
    say(wname, preset, "quantize", tuple(K.shape))
    tq.tq_quantize_kv(cb, dp, cache, K, V, torch.zeros(w.B, dtype=torch.int32, device="cuda"))
    say(wname, preset, "attend")
    out = tq.tq_attend_decode(cb, dp, cache, Q, torch.full((w.B,), T, dtype=torch.int32, device="cuda"), T)
    torch.cuda.synchronize()
    say(wname, preset, "device done")
    orc = H.make_oracle(preset)
    rng = np.random.default_rng(7)
    sample = np.unique(np.concatenate([np.arange(64), np.arange(T - 64, T), rng.integers(0, T, 16384)]))
    stats, errs = {}, []
    for b, h in [(0, 0), (w.B - 1, w.Hkv - 1)]:
        hc = {n: (None if t is None else t[b:b + 1, h:h + 1].cpu().numpy()) for n, t in cache.tensors().items()}
        kg = H.unpack_keys(orc, hc, 0, 0, T)
        vg = H.unpack_values(orc, hc, 0, 0, T)
        xk = K[b, h].float().cpu().numpy()
        xv = V[b, h].float().cpu().numpy()
        H.compare_keys(orc, xk[sample], {n: a[sample] for n, a in kg.items()}, stats)
        H.compare_values(orc, xv[sample], {n: a[sample] for n, a in vg.items()}, stats)
        hs = slice(h * w.G, (h + 1) * w.G)
        errs.append(H.compare_attention(orc, Q[b, hs].float().cpu().numpy(), kg, vg, T, out[b, hs].cpu().numpy()))
        say(wname, preset, "unit", (b, h), "checked")
    H.finish_stats(stats)
    say(wname, preset, "codes", stats, "max rel err", max(e["out"] for e in errs))


@pytest.mark.parametrize("preset", ["turbo2", "turbo3", "turbo4", "qjl1", "k8v4"])
def test_ragged_appends_and_canary(preset):
    """Bulk fill from unaligned starts, then one-token and block-crossing appends; slots never
    written keep their canary bytes."""
    B, Hkv, T_cap = 3, 2, 256
    cb, dp, cache = _setup(preset, B, Hkv, T_cap, zero=False)
    for t in cache.tensors().values():
        if t is not None:
            if t.dtype == torch.uint8:
                t.fill_(0xA5)
            else:
                t.fill_(0.5)
    rng = np.random.default_rng(7)
    starts = [0, 37, 64]
    # the last step writes row 0's last slot and skips rows 1 (negative start) and 2 (beyond T_cap)
    steps = [(150, starts), (1, [s + 150 for s in starts]), (5, [s + 151 for s in starts]),
             (1, [T_cap - 1, -1, T_cap + 3])]
    X = {"k": np.zeros((B, Hkv, T_cap, 128), np.float32), "v": np.zeros((B, Hkv, T_cap, 128), np.float32)}
    written = np.zeros((B, T_cap), dtype=bool)
    for n_new, st in steps:
        k = wl.round_to_bf16(rng.standard_normal((B, Hkv, n_new, 128)).astype(np.float32) * 3)
        v = wl.round_to_bf16(rng.standard_normal((B, Hkv, n_new, 128)).astype(np.float32))
        for b in range(B):
            if st[b] < 0 or st[b] + n_new > T_cap:
                assert n_new == 1  # rows that the call skips
                continue
            X["k"][b, :, st[b]:st[b] + n_new] = k[b]
            X["v"][b, :, st[b]:st[b] + n_new] = v[b]
            written[b, st[b]:st[b] + n_new] = True
        say("ragged", preset, "append", n_new, st)
        tq.tq_quantize_kv(cb, dp, cache, H.to_device(k, "bf16"), H.to_device(v, "bf16"),
                          torch.tensor(st, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    hc = H.cache_host(cache)
    orc = H.make_oracle(preset)
    canary = {name: np.full_like(a, 0xA5) for name, a in hc.items() if a is not None and a.dtype == np.uint8}
    stats = {}
    for b in range(B):
        wr = np.nonzero(written[b])[0]
        un = np.nonzero(~written[b])[0]
        for h in range(Hkv):
            kg = H.unpack_keys(orc, hc, b, h, T_cap)
            vg = H.unpack_values(orc, hc, b, h, T_cap)
            H.compare_keys(orc, X["k"][b, h, wr], {n: a[wr] for n, a in kg.items()}, stats)
            H.compare_values(orc, X["v"][b, h, wr], {n: a[wr] for n, a in vg.items()}, stats)
            # untouched slots
            assert np.all(hc["k_norm"][b, h, un] == 0.5) and np.all(hc["v_norm"][b, h, un] == 0.5)
            kc = H.unpack_keys(orc, {**hc, **canary}, b, h, T_cap)
            vc = H.unpack_values(orc, {**hc, **canary}, b, h, T_cap)
            if orc.k_bits:
                np.testing.assert_array_equal(kg["idx"][un], kc["idx"][un])
            if orc.k_qjl:
                np.testing.assert_array_equal(kg["sign"][un], kc["sign"][un])
            np.testing.assert_array_equal(vg["idx"][un], vc["idx"][un])
    H.finish_stats(stats)


def test_keys_only_and_values_only():
    """tq_quantize_kv with one tensor: a key-only 70-token append from unaligned starts (the
    general path), then a value-only one-token append (one workgroup per tile, the row's last
    slot included).  The written tensor matches the oracle; the other keeps its canary bytes."""
    preset = "turbo3"
    B, Hkv, T_cap = 2, 4, 128
    cb, dp, cache = _setup(preset, B, Hkv, T_cap, zero=False)
    for t in cache.tensors().values():
        if t is not None:
            t.fill_(0xA5) if t.dtype == torch.uint8 else t.fill_(0.5)
    rng = np.random.default_rng(13)
    k = wl.round_to_bf16(rng.standard_normal((B, Hkv, 70, 128)).astype(np.float32))
    v = wl.round_to_bf16(rng.standard_normal((B, Hkv, 1, 128)).astype(np.float32))
    k_st, v_st = [5, 0], [80, T_cap - 1]
    say("one-tensor", "keys", k_st)
    tq.tq_quantize_kv(cb, dp, cache, H.to_device(k, "bf16"), None, torch.tensor(k_st, dtype=torch.int32, device="cuda"))
    say("one-tensor", "values", v_st)
    tq.tq_quantize_kv(cb, dp, cache, None, H.to_device(v, "bf16"), torch.tensor(v_st, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    hc = H.cache_host(cache)
    orc = H.make_oracle(preset)
    canary = {name: np.full_like(a, 0xA5) for name, a in hc.items() if a is not None and a.dtype == np.uint8}
    stats = {}
    for b in range(B):
        kw = np.arange(k_st[b], k_st[b] + 70)
        k_un = np.setdiff1d(np.arange(T_cap), kw)
        v_un = np.setdiff1d(np.arange(T_cap), [v_st[b]])
        for h in range(Hkv):
            kg = H.unpack_keys(orc, hc, b, h, T_cap)
            vg = H.unpack_values(orc, hc, b, h, T_cap)
            H.compare_keys(orc, k[b, h], {n: a[kw] for n, a in kg.items()}, stats)
            H.compare_values(orc, v[b, h], {n: a[[v_st[b]]] for n, a in vg.items()}, stats)
            assert np.all(hc["k_norm"][b, h, k_un] == 0.5) and np.all(hc["v_norm"][b, h, v_un] == 0.5)
            kc = H.unpack_keys(orc, {**hc, **canary}, b, h, T_cap)
            vc = H.unpack_values(orc, {**hc, **canary}, b, h, T_cap)
            np.testing.assert_array_equal(kg["idx"][k_un], kc["idx"][k_un])
            np.testing.assert_array_equal(kg["sign"][k_un], kc["sign"][k_un])
            np.testing.assert_array_equal(vg["idx"][v_un], vc["idx"][v_un])
    H.finish_stats(stats)


@pytest.mark.parametrize("preset", ["turbo3", "turbo4"])
def test_many_units_partial_tiles(preset):
    """More tiles than persistent workgroups: a 100-token append from unaligned starts (partial
    first and last blocks, several tiles per workgroup, so the next tile's rows are prefetched
    across partial tiles), then a one-token append over 512 tiles (the general path, not the
    one-tile-per-workgroup one).  Every written vector is checked against the oracle; slots
    never written keep their canary bytes."""
    B, Hkv, T_cap = 4, 64, 256
    cb, dp, cache = _setup(preset, B, Hkv, T_cap, zero=False)
    for t in cache.tensors().values():
        if t is not None:
            t.fill_(0xA5) if t.dtype == torch.uint8 else t.fill_(0.5)
    rng = np.random.default_rng(11)
    X = {"k": np.zeros((B, Hkv, T_cap, 128), np.float32), "v": np.zeros((B, Hkv, T_cap, 128), np.float32)}
    written = np.zeros((B, T_cap), dtype=bool)
    starts = [37, 64, 101, 0]
    for n_new, st in [(100, starts), (1, [s + 100 for s in starts])]:
        k = wl.round_to_bf16(rng.standard_normal((B, Hkv, n_new, 128)).astype(np.float32) * 2)
        v = wl.round_to_bf16(rng.standard_normal((B, Hkv, n_new, 128)).astype(np.float32))
        for b in range(B):
            X["k"][b, :, st[b]:st[b] + n_new] = k[b]
            X["v"][b, :, st[b]:st[b] + n_new] = v[b]
            written[b, st[b]:st[b] + n_new] = True
        say("many-units", preset, "append", n_new, st)
        tq.tq_quantize_kv(cb, dp, cache, H.to_device(k, "bf16"), H.to_device(v, "bf16"),
                          torch.tensor(st, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    hc = H.cache_host(cache)
    orc = H.make_oracle(preset)
    canary = {name: np.full_like(a, 0xA5) for name, a in hc.items() if a is not None and a.dtype == np.uint8}
    stats = {}
    for b in range(B):
        wr = np.nonzero(written[b])[0]
        un = np.nonzero(~written[b])[0]
        for h in range(Hkv):
            kg = H.unpack_keys(orc, hc, b, h, T_cap)
            vg = H.unpack_values(orc, hc, b, h, T_cap)
            H.compare_keys(orc, X["k"][b, h, wr], {n: a[wr] for n, a in kg.items()}, stats)
            H.compare_values(orc, X["v"][b, h, wr], {n: a[wr] for n, a in vg.items()}, stats)
            assert np.all(hc["k_norm"][b, h, un] == 0.5) and np.all(hc["v_norm"][b, h, un] == 0.5)
            vc = H.unpack_values(orc, {**hc, **canary}, b, h, T_cap)
            np.testing.assert_array_equal(vg["idx"][un], vc["idx"][un])
    H.finish_stats(stats)
    say("many-units", preset, stats)


@pytest.mark.parametrize("preset,G", [("turbo3", 4), ("turbo4", 8), ("qjl1", 8), ("turbo3", 16)])
@pytest.mark.parametrize("repl", ["auto", "1"])
def test_attention_ragged_lengths(preset, G, repl):
    """Different sequence lengths per batch row (1, partial blocks, several slices)."""
    B, Hkv, T_cap = 4, 2, 2048
    cb, dp, cache = _setup(preset, B, Hkv, T_cap)
    rng = np.random.default_rng(11)
    K = wl.round_to_bf16(rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32) * 2)
    V = wl.round_to_bf16(rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32))
    Q = wl.round_to_bf16(rng.standard_normal((B, Hkv * G, 128)).astype(np.float32))
    start = torch.zeros(B, dtype=torch.int32, device="cuda")
    say("ragged-attn", preset, G, "quantize")
    tq.tq_quantize_kv(cb, dp, cache, H.to_device(K, "bf16"), H.to_device(V, "bf16"), start)
    lens = [1, 63, 1000, 2048]
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scores = torch.zeros((B, Hkv * G, T_cap), dtype=torch.float32, device="cuda")
    say("ragged-attn", preset, G, "attend", "tables", repl)
    with attention_tables(repl):
        out = tq.tq_attend_decode(cb, dp, cache, H.to_device(Q, "bf16"), seq, T_cap, scores_out=scores)
    torch.cuda.synchronize()
    hc, out, scores = H.cache_host(cache), out.cpu().numpy(), scores.cpu().numpy()
    orc = H.make_oracle(preset)
    for b in range(B):
        for h in range(Hkv):
            kg = H.unpack_keys(orc, hc, b, h, lens[b])
            vg = H.unpack_values(orc, hc, b, h, lens[b])
            hs = slice(h * G, (h + 1) * G)
            H.compare_attention(orc, Q[b, hs], kg, vg, lens[b], out[b, hs], scores[b, hs])
            # no score is written past the sequence length
            assert np.all(scores[b, hs, lens[b]:] == 0)


def test_attention_seq_len_clamped():
    """Sequence lengths outside 1..max_seq_len are clamped into it on the device: rows with
    lengths 0, -3 and beyond max_seq_len give bit for bit the outputs of lengths 1, 1 and
    max_seq_len, and a row inside the range is unaffected by its neighbours."""
    preset, G, B, Hkv, T_cap, max_len = "turbo3", 4, 4, 2, 1024, 700
    cb, dp, cache = _setup(preset, B, Hkv, T_cap)
    rng = np.random.default_rng(31)
    K = wl.round_to_bf16(rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32))
    V = wl.round_to_bf16(rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32))
    Q = H.to_device(wl.round_to_bf16(rng.standard_normal((B, Hkv * G, 128)).astype(np.float32)), "bf16")
    tq.tq_quantize_kv(cb, dp, cache, H.to_device(K, "bf16"), H.to_device(V, "bf16"),
                      torch.zeros(B, dtype=torch.int32, device="cuda"))
    say("seq-len clamp", "attend")
    got = tq.tq_attend_decode(cb, dp, cache, Q, torch.tensor([0, -3, 5000, 300], dtype=torch.int32, device="cuda"),
                              max_len)
    ref = tq.tq_attend_decode(cb, dp, cache, Q, torch.tensor([1, 1, max_len, 300], dtype=torch.int32, device="cuda"),
                              max_len)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    # and the clamped rows are attention over 1 and max_seq_len keys
    hc, out = H.cache_host(cache), ref.cpu().numpy()
    orc = H.make_oracle(preset)
    for b, T in ((0, 1), (2, max_len), (3, 300)):
        for h in range(Hkv):
            kg = H.unpack_keys(orc, hc, b, h, T)
            vg = H.unpack_values(orc, hc, b, h, T)
            hs = slice(h * G, (h + 1) * G)
            H.compare_attention(orc, Q[b, hs].cpu().float().numpy(), kg, vg, T,
                                out[b, hs])


@pytest.mark.parametrize("preset,G", [("turbo3", 4), ("turbo4", 8)])
def test_attention_softmax_scale_edges(preset, G):
    """Long per-wave streams (8 blocks per wave) through the online softmax's scale handling:
    row 0 has logits rising along the sequence (the running maximum moves in many blocks), row 1
    one key far above all others late in the sequence (a jump of the maximum by more than 2^32 in
    the log2 domain, after many blocks that kept their scale), row 2 value norms over eight
    decades (the weights' bound follows the value norms), row 3 plain Gaussian data."""
    B, Hkv, T = 4, 8, 32768
    cb, dp, cache = _setup(preset, B, Hkv, T)
    rng = np.random.default_rng(23)
    K = rng.standard_normal((B, Hkv, T, 128), dtype=np.float32)
    V = rng.standard_normal((B, Hkv, T, 128), dtype=np.float32)
    Q = wl.round_to_bf16(rng.standard_normal((B, Hkv * G, 128)).astype(np.float32))
    ramp = np.linspace(0.0, 40.0, T, dtype=np.float32)[:, None]
    for h in range(Hkv):
        u = Q[0, h * G] / np.linalg.norm(Q[0, h * G])
        K[0, h] += ramp * u[None, :]
        u1 = Q[1, h * G] / np.linalg.norm(Q[1, h * G])
        K[1, h, (8 * T) // 10] = 60.0 * u1 * math.sqrt(128)
    V[2] *= (10.0 ** rng.uniform(-4.0, 4.0, size=(Hkv, T, 1))).astype(np.float32)
    K, V = wl.round_to_bf16(K), wl.round_to_bf16(V)
    start = torch.zeros(B, dtype=torch.int32, device="cuda")
    say("scale-edges", preset, G, "quantize")
    tq.tq_quantize_kv(cb, dp, cache, H.to_device(K, "bf16"), H.to_device(V, "bf16"), start)
    seq = torch.full((B,), T, dtype=torch.int32, device="cuda")
    say("scale-edges", preset, G, "attend")
    out = tq.tq_attend_decode(cb, dp, cache, H.to_device(Q, "bf16"), seq, T)
    torch.cuda.synchronize()
    hc, out = H.cache_host(cache), out.cpu().numpy()
    orc = H.make_oracle(preset)
    for b in range(B):
        for h in (0, 5):
            kg = H.unpack_keys(orc, hc, b, h, T)
            vg = H.unpack_values(orc, hc, b, h, T)
            hs = slice(h * G, (h + 1) * G)
            H.compare_attention(orc, Q[b, hs], kg, vg, T, out[b, hs])


@pytest.mark.parametrize("B,G,T_cap,lens", [(2, 8, 10240, [10240, 3001]), (1, 8, 40960, [40960 - 100]),
                                            (1, 4, 262144, [262144 - 37])])
def test_attention_merge_levels(B, G, T_cap, lens):
    """Context splits of several sizes with the default merge groups of 16 slices: 10 slices
    (one merge group, the second row leaving most slices empty), 40 slices (groups of 16, 16
    and 8), and 256 slices (16 groups of 16).  A second call with the same workspace must give
    identical outputs (the arrival counters are reset per call)."""
    _merge_case(B, G, T_cap, lens)


@pytest.mark.parametrize("mgroup", [1, 32])
def test_attention_merge_group_sizes(mgroup):
    """TQ_ATTN_MGROUP at both ends of its range.  The library reads it once per process, so
    the cases run in a child process.  1: 10 slices form 10 groups of one slice and 40 slices
    form 20 groups of two (the group grows to keep at most 32 groups); 32: 10 slices form one
    group, 40 slices groups of 32 and 8."""
    import os
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("from tests.test_gpu_parity import _merge_case; "
            "_merge_case(2, 8, 10240, [10240, 3001]); _merge_case(1, 8, 40960, [40960 - 100])")
    say("merge group size", mgroup, "in a child process")
    r = subprocess.run([sys.executable, "-u", "-c", code], cwd=root, timeout=100,
                       env=dict(os.environ, TQ_ATTN_MGROUP=str(mgroup)))
    assert r.returncode == 0, f"child exited with {r.returncode}"


def _merge_case(B, G, T_cap, lens):
    preset, Hkv = "turbo3", 1
    cb, dp, cache = _setup(preset, B, Hkv, T_cap)
    rng = np.random.default_rng(13)
    K = wl.round_to_bf16(rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32) * 2)
    V = wl.round_to_bf16(rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32))
    Q = wl.round_to_bf16(rng.standard_normal((B, Hkv * G, 128)).astype(np.float32))
    say("merge-levels", B, G, T_cap, "quantize")
    tq.tq_quantize_kv(cb, dp, cache, H.to_device(K, "bf16"), H.to_device(V, "bf16"),
                      torch.zeros(B, dtype=torch.int32, device="cuda"))
    del K, V
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scores = torch.zeros((B, Hkv * G, T_cap), dtype=torch.float32, device="cuda")
    ws = torch.zeros(tq.attend_workspace_bytes(cb, dp, cache, Hkv * G, T_cap), dtype=torch.uint8, device="cuda")
    qd = H.to_device(Q, "bf16")
    say("merge-levels", B, G, T_cap, "attend x2")
    out1 = tq.tq_attend_decode(cb, dp, cache, qd, seq, T_cap, scores_out=scores, workspace=ws).clone()
    out2 = tq.tq_attend_decode(cb, dp, cache, qd, seq, T_cap, workspace=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out1.cpu().numpy(), out2.cpu().numpy())
    hc, out, scores = H.cache_host(cache), out1.cpu().numpy(), scores.cpu().numpy()
    orc = H.make_oracle(preset)
    for b in range(B):
        kg = H.unpack_keys(orc, hc, b, 0, lens[b])
        vg = H.unpack_values(orc, hc, b, 0, lens[b])
        e = H.compare_attention(orc, Q[b], kg, vg, lens[b], out[b], scores[b])
        say("merge-levels", b, lens[b], e)


# Bit widths beyond turbo3/turbo4/qjl1 (the same kernels with other code widths): MSE-only
# keys without the sketch, 1- and 4-bit key codes with and without it, 1-bit values, and
# asymmetric key/value widths, at each group size.
@pytest.mark.parametrize("preset,G,dtype", [("turbo3", 4, "bf16"), ("turbo4", 8, "bf16"), ("qjl1", 16, "f32"),
                                            ("k8v4", 8, "bf16")])
def test_hadamard_rotation(preset, G, dtype):
    """The randomized Walsh-Hadamard rotation mode: same kernels, parameters from the other
    builder; codes, scores and outputs against the oracle in that mode (bf16 and fp32 inputs)."""
    B, Hkv, T_cap = 1, 2, 3072
    lens = [3000]
    cb, dp, cache = _setup(preset, B, Hkv, T_cap, seed=4, rotation="hadamard")
    rng = np.random.default_rng(31)
    K = rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32) * 1.5
    V = rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32)
    Q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float32)
    if dtype == "bf16":
        K, V, Q = wl.round_to_bf16(K), wl.round_to_bf16(V), wl.round_to_bf16(Q)
    say("hadamard", preset, G, dtype, "quantize")
    tq.tq_quantize_kv(cb, dp, cache, H.to_device(K, dtype), H.to_device(V, dtype),
                      torch.zeros(B, dtype=torch.int32, device="cuda"))
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scores = torch.zeros((B, Hkv * G, T_cap), dtype=torch.float32, device="cuda")
    say("hadamard", preset, G, dtype, "attend")
    out = tq.tq_attend_decode(cb, dp, cache, H.to_device(Q, dtype), seq, T_cap, scores_out=scores)
    torch.cuda.synchronize()
    hc, out, scores = H.cache_host(cache), out.cpu().numpy(), scores.cpu().numpy()
    orc = H.make_oracle(preset, seed=4, rotation="hadamard")
    stats = {}
    for h in range(Hkv):
        kg = H.unpack_keys(orc, hc, 0, h, lens[0])
        vg = H.unpack_values(orc, hc, 0, h, lens[0])
        H.compare_keys(orc, K[0, h, :lens[0]], kg, stats)
        H.compare_values(orc, V[0, h, :lens[0]], vg, stats)
        hs = slice(h * G, (h + 1) * G)
        H.compare_attention(orc, Q[0, hs], kg, vg, lens[0], out[0, hs], scores[0, hs])
    H.finish_stats(stats)
    say("hadamard", preset, G, dtype, "codes", stats)


@pytest.mark.parametrize("cfg,G", [((1, 1, 2), 4), ((2, 0, 3), 8), ((3, 0, 4), 16), ((1, 0, 1), 8),
                                   ((4, 1, 4), 4), ((4, 0, 2), 16), ((4, 1, 1), 8), ((1, 1, 4), 16),
                                   ((0, 1, 1), 4), ((2, 1, 1), 16),
                                   ((8, 0, 4), 4), ((8, 1, 4), 8), ((5, 1, 3), 16), ((6, 0, 2), 8),
                                   ((7, 1, 4), 4), ((8, 0, 4), 16), ((5, 0, 1), 4), ((6, 1, 2), 4)])
@pytest.mark.parametrize("repl", ["auto", "1"])
def test_bit_mix_variants(cfg, G, repl):
    B, Hkv, T_cap = 2, 2, 4096
    lens = [4096, 2500]
    cb, dp, cache = _setup(cfg, B, Hkv, T_cap)
    rng = np.random.default_rng(100 * cfg[0] + 10 * cfg[1] + cfg[2])
    K = wl.round_to_bf16(rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32) * 2)
    V = wl.round_to_bf16(rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32))
    Q = wl.round_to_bf16(rng.standard_normal((B, Hkv * G, 128)).astype(np.float32))
    say("bit-mix", cfg, G, "quantize")
    tq.tq_quantize_kv(cb, dp, cache, H.to_device(K, "bf16"), H.to_device(V, "bf16"),
                      torch.zeros(B, dtype=torch.int32, device="cuda"))
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scores = torch.zeros((B, Hkv * G, T_cap), dtype=torch.float32, device="cuda")
    say("bit-mix", cfg, G, "attend", "tables", repl)
    with attention_tables(repl):
        out = tq.tq_attend_decode(cb, dp, cache, H.to_device(Q, "bf16"), seq, T_cap, scores_out=scores)
    torch.cuda.synchronize()
    hc, out, scores = H.cache_host(cache), out.cpu().numpy(), scores.cpu().numpy()
    orc = H.make_oracle(cfg)
    stats = {}
    for b in range(B):
        for h in range(Hkv):
            kg = H.unpack_keys(orc, hc, b, h, lens[b])
            vg = H.unpack_values(orc, hc, b, h, lens[b])
            H.compare_keys(orc, K[b, h, :lens[b]], kg, stats)
            H.compare_values(orc, V[b, h, :lens[b]], vg, stats)
            hs = slice(h * G, (h + 1) * G)
            H.compare_attention(orc, Q[b, hs], kg, vg, lens[b], out[b, hs], scores[b, hs])
    H.finish_stats(stats)
    say("bit-mix", cfg, G, "codes", stats)


@pytest.mark.parametrize("preset,G,dtype,lens", [("turbo3", 4, "bf16", [1500, 900]), ("turbo4", 8, "f32", [1500, 900]),
                                                  ("qjl1", 16, "bf16", [1500, 900]), ("turbo4", 4, "bf16", [0, 63]),
                                                  ("turbo3", 8, "bf16", [64, 2047]), ("turbo2", 16, "bf16", [640, 1]),
                                                  ("k8v4", 8, "bf16", [1500, 900]), ((7, 1, 4), 4, "f32", [63, 1000])])
def test_decode_step_matches_separate_calls(preset, G, dtype, lens):
    """tq_decode_step (new token + query rotation in one launch, then attention) gives the same
    cache bytes and bit-identical outputs as tq_quantize_kv followed by tq_attend_decode, and
    its output matches the oracle; new tokens mid-block, in block 0, at a block start and in
    the last slot."""
    B, Hkv, T_cap = 2, 2, 2048
    rng = np.random.default_rng(41)
    K = rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32)
    Q = rng.standard_normal((B, Hkv * G, 128)).astype(np.float32)
    if dtype == "bf16":
        K, V, Q = wl.round_to_bf16(K), wl.round_to_bf16(V), wl.round_to_bf16(Q)
    caches = []
    for _ in range(2):
        cb, dp, cache = _setup(preset, B, Hkv, T_cap)
        # prefill: the first lens[b] tokens (the rest of each row is written but not attended)
        tq.tq_quantize_kv(cb, dp, cache, H.to_device(K, dtype), H.to_device(V, dtype),
                          torch.zeros(B, dtype=torch.int32, device="cuda"))
        caches.append(cache)
    # row b's new token is token lens[b] of the host arrays
    k1 = torch.stack([H.to_device(K[b, :, lens[b]:lens[b] + 1], dtype) for b in range(B)])
    v1 = torch.stack([H.to_device(V[b, :, lens[b]:lens[b] + 1], dtype) for b in range(B)])
    start = torch.tensor(lens, dtype=torch.int32, device="cuda")
    seq = torch.tensor([n + 1 for n in lens], dtype=torch.int32, device="cuda")
    qd = H.to_device(Q, dtype)
    say("decode-step", preset, G, dtype, "separate calls")
    tq.tq_quantize_kv(cb, dp, caches[0], k1, v1, start)
    out_a = tq.tq_attend_decode(cb, dp, caches[0], qd, seq, T_cap).clone()
    say("decode-step", preset, G, dtype, "fused step")
    out_b = tq.tq_decode_step(cb, dp, caches[1], k1, v1, start, qd, seq, T_cap)
    torch.cuda.synchronize()
    for name, t in caches[0].tensors().items():
        if t is not None:
            assert torch.equal(t, caches[1].tensors()[name]), name
    np.testing.assert_array_equal(out_a.cpu().numpy(), out_b.cpu().numpy())
    hc, out = H.cache_host(caches[1]), out_b.cpu().numpy()
    orc = H.make_oracle(preset)
    for b in range(B):
        for h in range(Hkv):
            n = lens[b] + 1
            kg = H.unpack_keys(orc, hc, b, h, n)
            vg = H.unpack_values(orc, hc, b, h, n)
            hs = slice(h * G, (h + 1) * G)
            H.compare_attention(orc, Q[b, hs], kg, vg, n, out[b, hs], None)


@pytest.mark.parametrize("G", [4, 8, 16])
def test_bf16_baseline(G):
    """The uncompressed bf16 baseline against plain softmax attention in fp64 (bf16-rounded
    inputs).  Its softmax weights enter the value products as bf16, so outputs agree to the
    bf16 unit roundoff (2^-8) relative to the output's largest magnitude."""
    B, Hkv, T_cap = 2, 2, 2048
    lens = [2048, 777]
    rng = np.random.default_rng(50 + G)
    K = wl.round_to_bf16(rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32))
    V = wl.round_to_bf16(rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32))
    Q = wl.round_to_bf16(rng.standard_normal((B, Hkv * G, 128)).astype(np.float32))
    kd, vd, qd = (H.to_device(x, "bf16") for x in (K, V, Q))
    say("bf16-baseline", G)
    out = tq.tq_bf16_attend_decode(kd, tq.bf16_value_chunks(vd), qd, torch.tensor(lens, dtype=torch.int32,
                                                                               device="cuda"), T_cap)
    out = out.cpu().numpy()
    for b in range(B):
        for h in range(Hkv * G):
            k = K[b, h // G, :lens[b]].astype(np.float64)
            v = V[b, h // G, :lens[b]].astype(np.float64)
            s = k @ Q[b, h].astype(np.float64) / np.sqrt(128.0)
            p = np.exp(s - s.max())
            ref = (p / p.sum()) @ v
            assert np.abs(out[b, h] - ref).max() <= 2.0 ** -8 * np.abs(ref).max(), (b, h)


def test_special_vectors():
    """Zero vectors, one-hot vectors, huge and tiny magnitudes, fp32 inputs."""
    preset = "turbo3"
    T = 128
    cb, dp, cache = _setup(preset, 1, 1, T)
    rng = np.random.default_rng(5)
    K = rng.standard_normal((1, 1, T, 128)).astype(np.float32)
    K[0, 0, 0] = 0
    K[0, 0, 1] = 0
    K[0, 0, 1, 17] = 1.0
    K[0, 0, 2] *= 1e30
    K[0, 0, 3] *= 1e-30
    K[0, 0, 4] = 1.0
    V = K.copy()
    say("special", "quantize")
    tq.tq_quantize_kv(cb, dp, cache, H.to_device(K, "f32"), H.to_device(V, "f32"),
                      torch.zeros(1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    hc = H.cache_host(cache)
    orc = H.make_oracle(preset)
    stats = {}
    kg = H.unpack_keys(orc, hc, 0, 0, T)
    vg = H.unpack_values(orc, hc, 0, 0, T)
    H.compare_keys(orc, K[0, 0].astype(np.float64), kg, stats)
    H.compare_values(orc, V[0, 0].astype(np.float64), vg, stats)
    assert kg["n"][0] == 0 and np.all(kg["idx"][0] == 2) and kg["gamma"][0] == 0 and np.all(kg["sign"][0])
    assert np.all(vg["idx"][0] == 4)


def test_deterministic():
    preset = "turbo3"
    B, Hkv, T = 2, 2, 1024
    rng = np.random.default_rng(1)
    K = H.to_device(wl.round_to_bf16(rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)), "bf16")
    V = H.to_device(wl.round_to_bf16(rng.standard_normal((B, Hkv, T, 128)).astype(np.float32)), "bf16")
    Q = H.to_device(wl.round_to_bf16(rng.standard_normal((B, Hkv * 4, 128)).astype(np.float32)), "bf16")
    outs = []
    for rep in range(2):
        cb, dp, cache = _setup(preset, B, Hkv, T)
        say("determinism", rep)
        tq.tq_quantize_kv(cb, dp, cache, K, V, torch.zeros(B, dtype=torch.int32, device="cuda"))
        out = tq.tq_attend_decode(cb, dp, cache, Q, torch.full((B,), T, dtype=torch.int32, device="cuda"), T)
        torch.cuda.synchronize()
        outs.append((H.cache_host(cache), out.cpu().numpy()))
    for name, a in outs[0][0].items():
        if a is not None:
            np.testing.assert_array_equal(a, outs[1][0][name])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def _prefill_case(preset, B, Hkv, G, T_cap, T_q, starts, dtype, seed, check_units=None, sample=None):
    """Bulk-quantize T_cap tokens, run causal prefill attention of T_q queries per row starting at
    position starts[b], and compare the checked (row, kv-head) units with the oracle on the
    GPU-written cache (every query, or the query indices in `sample`)."""
    cb, dp, cache = _setup(preset, B, Hkv, T_cap)
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32) * 2
    V = rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32)
    Q = rng.standard_normal((B, Hkv * G, T_q, 128)).astype(np.float32)
    if dtype == "bf16":
        K, V, Q = wl.round_to_bf16(K), wl.round_to_bf16(V), wl.round_to_bf16(Q)
    say("prefill", preset, B, Hkv, G, T_cap, T_q, starts, "quantize")
    tq.tq_quantize_kv(cb, dp, cache, H.to_device(K, dtype), H.to_device(V, dtype),
                      torch.zeros(B, dtype=torch.int32, device="cuda"))
    del K, V
    say("prefill", preset, "attend")
    out = tq.tq_attend_prefill(cb, dp, cache, H.to_device(Q, dtype), torch.tensor(starts, dtype=torch.int32,
                                                                                  device="cuda"), T_cap)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    orc = H.make_oracle(preset)
    units = check_units or [(b, h) for b in range(B) for h in range(Hkv)]
    idx = np.arange(T_q) if sample is None else np.asarray(sample)
    worst = 0.0
    for b, h in units:
        hc = {n: (None if t is None else t[b:b + 1, h:h + 1].cpu().numpy()) for n, t in cache.tensors().items()}
        pos = starts[b] + idx
        T = int(pos.max()) + 1
        kg = H.unpack_keys(orc, hc, 0, 0, T)
        vg = H.unpack_values(orc, hc, 0, 0, T)
        hs = slice(h * G, (h + 1) * G)
        _, ref = orc.attend_prefill(Q[b, hs][:, idx].astype(np.float64), kg, vg, pos)
        got = out[b, hs][:, idx]
        d = np.abs(got - ref).max(axis=2)
        mag = np.abs(ref).max(axis=2)
        err = float((d / np.maximum(mag, 1e-300)).max())
        worst = max(worst, err)
        H.record("out_err_vs_max", err)
        assert np.all(d <= H.SCORE_TOL * mag), ("prefill outputs", (b, h), err)
    say("prefill", preset, "max rel err", worst)


@pytest.mark.parametrize("preset,G,dtype,T_q,starts", [("turbo3", 4, "bf16", 300, [0, 100]),
                                                       ("turbo4", 8, "f32", 257, [0, 37]),
                                                       ("qjl1", 16, "bf16", 130, [5, 0]),
                                                       ((2, 0, 3), 4, "bf16", 70, [1, 64]),
                                                       ("turbo3", 4, "bf16", 1, [0, 400]),
                                                       ("k8v4", 4, "bf16", 200, [0, 50]),
                                                       ((6, 1, 4), 8, "f32", 100, [3, 0])])
def test_prefill_matches_oracle(preset, G, dtype, T_q, starts):
    """Causal prefill attention over the packed cache (tq_attend_prefill): ragged prompt lengths,
    prompts that start after an earlier context, a single query, every query column compared
    with the oracle's causal attention on the GPU-written cache."""
    _prefill_case(preset, 2, 2, G, 512, T_q, starts, dtype, seed=60 + T_q)


def test_prefill_4k_prompt():
    """A 4096-token prompt at the Llama-3.1-8B layer shape (32 q-heads, 8 kv-heads), every query of
    two kv-heads checked."""
    _prefill_case("turbo3", 1, 8, 4, 4096, 4096, [0], "bf16", seed=71, check_units=[(0, 0), (0, 7)])


def test_prefill_32k_prompt_sampled():
    """A 32768-token prompt at the Llama-3.1-8B layer shape, queries sampled (first and last 64,
    block edges and 200 random positions) for two kv-heads."""
    T = 32768
    rng = np.random.default_rng(5)
    sample = np.unique(np.concatenate([np.arange(64), np.arange(T - 64, T), [4095, 4096, 16383, 16384],
                                       rng.integers(0, T, 200)]))
    _prefill_case("turbo3", 1, 8, 4, T, T, [0], "bf16", seed=72, check_units=[(0, 0), (0, 5)], sample=sample)
