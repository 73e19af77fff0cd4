"""Pins for the oracle's packing layout and the pages' bits-per-weight ledgers."""
import numpy as np
import pytest

import oracle


def test_hand_examples(golden):
    g = golden("pack_layout.txt")
    c2 = np.array(g["codes_2bit"], dtype=np.int64)[None, :]
    c3 = np.array(g["codes_3bit"], dtype=np.int64)[None, :]
    s = np.array(g["scales"])[None, :]
    buf2 = oracle.pack(c2, s, 2, 4)
    assert buf2[:2].tolist() == [int(v) for v in g["bytes_2bit"]]
    assert buf2[2:].tolist() == [int(v) for v in g["scale_bytes"]]
    buf3 = oracle.pack(c3, s, 3, 4)
    assert buf3[:3].tolist() == [int(v) for v in g["bytes_3bit"]]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_roundtrip_and_size(bits):
    rng = np.random.default_rng(40 + bits)
    rows, n, g = 7, 64, 16
    codes = rng.integers(0, 2 ** bits, size=(rows, n))
    scales = oracle.fp16_rne(rng.uniform(-1, 1, size=(rows, n // g)))
    buf = oracle.pack(codes, scales, bits, g)
    assert buf.shape[0] == rows * n * bits // 8 + 2 * rows * (n // g) == oracle.packed_bytes(rows, n, bits, g)
    c2, s2 = oracle.unpack(buf, rows, n, bits, g)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_bit_positions_by_bruteforce():
    rng = np.random.default_rng(45)
    for bits in (2, 3):
        codes = rng.integers(0, 2 ** bits, size=(3, 24))
        buf = oracle.pack(codes, np.ones((3, 1)), bits, 24)
        nb = 24 * bits // 8
        for r in range(3):
            for j in range(24):
                v = 0
                for i in range(bits):
                    pos = j * bits + i
                    v |= ((int(buf[r * nb + pos // 8]) >> (pos % 8)) & 1) << i
                assert v == codes[r, j]


def test_pages_ledgers(golden):
    g = golden("ledger_recipe.txt")
    # the parts add up to the printed totals (the Qwen3-4B card rounds 2.639 to 2.638)
    assert abs(g["qwen_code_bpw"][0] + g["qwen_scale_bpw"][0] - g["qwen_total_bpw"][0]) <= 0.0015
    assert abs(g["a1_code_bpw"][0] + g["a1_scale_bpw"][0] - g["a1_total_bpw"][0]) <= 1e-9
    # container bytes ~= weights x b/w / 8
    for p in ("qwen", "a1"):
        gib = g[p + "_weights"][0] * g[p + "_total_bpw"][0] / 8 / 2 ** 30
        assert abs(gib - g[p + "_container_gib"][0]) < 0.01


def test_ledger_of_this_layout():
    # a 4096 x 2560 module at 2 bits with one fp16 scale per 64 weights: 2 + 16/64 = 2.25 b/w
    total, code, scale = oracle.ledger_bits_per_weight(4096 * 2560, 2 * 4096 * 2560, 4096 * 40)
    assert (code, scale, total) == (2.0, 0.25, 2.25)
    assert oracle.packed_bytes(4096, 2560, 2, 64) * 8 / (4096 * 2560) == 2.25
