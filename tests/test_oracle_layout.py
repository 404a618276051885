"""Pins of the packed-cache layout oracle: hand-derived bytes, round trips, byte accounting."""
import os

import numpy as np
import pytest

from oracle import layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    out = []
    for line in open(os.path.join(GOLDEN, "layout_cases.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, tail = line.split(":")
        kind, bits, T, tok, coord, code = head.split()
        expect = {int(a): int(b) for a, b in (kv.split("=") for kv in tail.split())}
        out.append((kind, int(bits), int(T), int(tok), int(coord), int(code), expect))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}{c[1]}-t{c[3]}-j{c[4]}")
def test_hand_derived_positions(case):
    kind, bits, T, tok, coord, code, expect = case
    codes = np.zeros((T, 128), dtype=np.int64)
    codes[tok, coord] = code
    packed = layout.pack(codes.astype(bool) if kind == "s" else codes, bits, kind).ravel()
    nz = {int(i): int(packed[i]) for i in np.nonzero(packed)[0]}
    assert nz == expect
    back = layout.unpack(packed.reshape(-1, 1024 * bits), T, 128, bits, kind)
    np.testing.assert_array_equal(back.astype(np.int64), codes)


@pytest.mark.parametrize("kind,bits", [("k", 1), ("k", 2), ("k", 3), ("k", 4), ("k", 5), ("k", 7), ("k", 8), ("s", 1),
                                       ("v", 1), ("v", 2), ("v", 3), ("v", 4)])
@pytest.mark.parametrize("T", [1, 64, 150])
def test_round_trip(kind, bits, T):
    rng = np.random.default_rng(T * 10 + bits)
    hi = 2 if kind == "s" else (1 << bits)
    codes = rng.integers(0, hi, size=(T, 128))
    if kind == "s":
        codes = codes.astype(bool)
    packed = layout.pack(codes, bits, kind)
    assert packed.shape == (layout.n_blocks(T), 1024 * (1 if kind == "s" else bits))
    back = layout.unpack(packed, T, 128, bits, kind)
    np.testing.assert_array_equal(back, codes if kind == "s" else codes.astype(np.uint8))


@pytest.mark.parametrize("kind,bits", [("k", 2), ("k", 3), ("k", 6), ("k", 8), ("v", 3), ("v", 4), ("s", 1)])
def test_layout_is_a_bijection(kind, bits):
    # every bit of a full block is used exactly once
    T = 64
    off = layout._offsets(kind, T, 128, 1 if kind == "s" else bits)
    b = 1 if kind == "s" else bits
    allbits = (off[..., None] + np.arange(b)).ravel()
    assert len(np.unique(allbits)) == T * 128 * b == 1024 * b * 8
    assert allbits.min() == 0 and allbits.max() == 1024 * b * 8 - 1


def test_tokens_own_whole_words_for_keys():
    # every 32-bit word of a key-code or sign block belongs to a single token, so a
    # one-token append never shares a word with another token
    for kind, bits in [("k", 2), ("k", 3), ("s", 1)]:
        off = layout._offsets(kind, 64, 128, bits)
        b = bits
        words = (off[..., None] + np.arange(b)) // 32
        owner = {}
        for tok in range(64):
            for w in np.unique(words[tok]):
                assert owner.setdefault(int(w), tok) == tok


def test_byte_accounting_matches_pages():
    # "52 bytes per 128 values" at 3 bits and compression 4.9x / 3.8x versus FP16
    # (page "Google TurboQuant простыми словами", section "Бенчмарки TurboQuant").
    figs = {}
    for line in open(os.path.join(GOLDEN, "pages_figures.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()[:2]
            figs[k] = float(v)
    v3 = layout.bytes_per_token(2, 1, 3)["v"]
    v4 = layout.bytes_per_token(3, 1, 4)["v"]
    assert v3 == figs["block_bytes_3bit"]
    assert round(2 * figs["block_values"] / v3, 1) == figs["ratio_3bit_vs_fp16"]
    assert round(2 * figs["block_values"] / v4, 1) == figs["ratio_4bit_vs_fp16"]
    assert layout.bytes_per_token(2, 1, 3)["total"] == 108
    assert layout.bytes_per_token(3, 1, 4)["total"] == 140
    assert layout.bytes_per_token(0, 1, 3)["total"] == 72
