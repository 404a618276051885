"""tq_attend_decode_noalloc (attention whose workspace is the library's fixed device scratch)
against tq_attend_decode with a caller workspace: two calls in a row on the same GPU, the
second with a smaller input (fewer batch rows, heads and keys), each bit-identical to the
entry point with a workspace (same kernels, same context split), and within the parity bar
of the oracle.  A call too large for the scratch fails before any launch."""
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


def _case(preset, B, Hkv, G, T_cap, lens, seed):
    cb = tq.tq_build_codebook(*wl.PRESETS[preset], seed=0)
    dp = tq.upload_params(cb)
    cache = tq.KVCache(cb, B, Hkv, T_cap)
    rng = np.random.default_rng(seed)
    K = wl.round_to_bf16(rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32) * 2)
    V = wl.round_to_bf16(rng.standard_normal((B, Hkv, T_cap, 128)).astype(np.float32))
    Q = wl.round_to_bf16(rng.standard_normal((B, Hkv * G, 128)).astype(np.float32))
    tq.tq_quantize_kv(cb, dp, cache, H.to_device(K, "bf16"), H.to_device(V, "bf16"),
                      torch.zeros(B, dtype=torch.int32, device="cuda"))
    return cb, dp, cache, Q, torch.tensor(lens, dtype=torch.int32, device="cuda")


def test_noalloc_matches_workspace_entry_point_twice():
    cases = [("turbo3", 4, 8, 4, 8192, [8192, 5000, 64, 1], 3),  # larger first
             ("turbo4", 1, 2, 8, 1024, [777], 4)]                # then smaller: fewer rows, heads, keys
    for preset, B, Hkv, G, T_cap, lens, seed in cases:
        cb, dp, cache, Q, seq = _case(preset, B, Hkv, G, T_cap, lens, seed)
        qd = H.to_device(Q, "bf16")
        say("no-alloc", preset, B, Hkv, G, T_cap, lens)
        ref = tq.tq_attend_decode(cb, dp, cache, qd, seq, T_cap).clone()
        got = tq.tq_attend_decode_noalloc(cb, dp, cache, qd, seq, T_cap)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), ref.cpu().numpy())
        # and the parity bar against the oracle for every (batch row, kv-head)
        hc, out = H.cache_host(cache), got.cpu().numpy()
        orc = H.make_oracle(preset)
        for b in range(B):
            for h in range(Hkv):
                kg = H.unpack_keys(orc, hc, b, h, lens[b])
                vg = H.unpack_values(orc, hc, b, h, lens[b])
                hs = slice(h * G, (h + 1) * G)
                H.compare_attention(orc, Q[b, hs], kg, vg, lens[b], out[b, hs], None)


def test_noalloc_rejects_a_call_beyond_its_scratch():
    # 1024 x 32 q-heads of query records alone need 32 MiB, beyond the 16 MiB scratch
    cb = tq.tq_build_codebook(*wl.PRESETS["turbo3"], seed=0)
    dp = tq.upload_params(cb)
    cache = tq.KVCache(cb, 1024, 8, 64)
    q = torch.zeros((1024, 32, 128), dtype=torch.bfloat16, device="cuda")
    seq = torch.ones(1024, dtype=torch.int32, device="cuda")
    with pytest.raises(tq.TQError, match="TQ_ERR_WORKSPACE"):
        tq.tq_attend_decode_noalloc(cb, dp, cache, q, seq, 64)
