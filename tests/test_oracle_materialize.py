"""Pins for the oracle's materializer (Wringer model cards, "What is in this repo" and "Honest
caveats": packed module -> fake-quant bf16 weights at ledger precision)."""
import numpy as np
import torch

import oracle


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-6, 6, 20000).astype(np.float32)
    # exact halfway cases: 8 significant bits plus a trailing half ulp, both parities
    base = np.float32(1.0) + np.arange(0, 256, dtype=np.float32) * np.float32(2.0 ** -7)
    ties = base + np.float32(2.0 ** -8)
    x = np.concatenate([x, ties, -ties, [0.0, -0.0]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = oracle.bf16_rne_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_rounding_is_a_single_rounding():
    # 1 + 2^-8 + 2^-30 lies just above the midpoint of 1 and 1 + 2^-7: one rounding gives
    # 1 + 2^-7; rounding to fp32 first would land exactly on the midpoint and tie to 1.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.bf16_rne_bits(np.array([x]))[0] == 0x3F81
    assert oracle.bf16_rne_bits(np.array([np.float64(np.float32(x))]))[0] == 0x3F80


def _module(rng, rows, n, bits, group, pow2_scales):
    L = 2 ** bits - 1
    codes = rng.integers(0, L + 1, size=(rows, n))
    if pow2_scales:
        scales = 2.0 ** rng.integers(-9, -3, size=(rows, n // group)).astype(np.float64)
    else:
        scales = oracle.fp16_rne(rng.uniform(1e-3, 2e-2, size=(rows, n // group)))
    return codes, scales, oracle.pack(codes, scales, bits, group)


def test_materialize_without_rotation_is_the_dequantized_weights():
    rng = np.random.default_rng(7)
    rows, n, bits, g = 6, 256, 3, 32
    codes, scales, buf = _module(rng, rows, n, bits, g, pow2_scales=True)
    got = oracle.bf16_bits_to_f64(oracle.materialize(buf, rows, n, bits, g, 0, None, 200))
    # power-of-two scales times odd levels below 8 have at most 3 significant bits: exact in bf16
    assert np.array_equal(got, oracle.dequant(codes, scales, bits, g)[:, :200])


def test_materialize_undoes_the_rotation():
    rng = np.random.default_rng(8)
    rows, n, bits, g, m = 5, 512, 2, 64, 128
    signs = rng.choice([-1.0, 1.0], size=n)
    codes, scales, buf = _module(rng, rows, n, bits, g, pow2_scales=False)
    exact = oracle.materialize_exact(buf, rows, n, bits, g, m, signs, n)
    assert np.allclose(oracle.rotate_rows(exact, m, signs), oracle.dequant(codes, scales, bits, g), atol=1e-15)
    got = oracle.bf16_bits_to_f64(oracle.materialize(buf, rows, n, bits, g, m, signs, n))
    # one rounding: within half a bf16 ulp of the exact weights (x = f 2^e, f in [0.5, 1):
    # the ulp is 2^(e - 8))
    _, e = np.frexp(exact)
    assert np.all(np.abs(got - exact) <= np.ldexp(1.0, e - 9))


def test_materialize_keeps_exact_cancellations_zero():
    # a block of equal dequantized values: H_m v is m v_0 in the first entry and exactly zero
    # in every other one, so the materialized weights there are +-0 (a normalised fp64
    # product leaves residues near 1e-17 that bf16 would keep)
    rows, n, bits, g, m = 3, 64, 4, 32, 32
    L = 2 ** bits - 1
    codes = np.full((rows, n), 11)
    scales = oracle.fp16_rne(np.array([[0.0123, 0.0071]] * rows))
    buf = oracle.pack(codes, scales, bits, g)
    signs = np.random.default_rng(9).choice([-1.0, 1.0], size=n)
    got = oracle.bf16_bits_to_f64(oracle.materialize(buf, rows, n, bits, g, m, signs, n))
    first = np.zeros(n, dtype=bool)
    first[[0, 32]] = True
    assert np.all(got[:, ~first] == 0.0)
    lead = (2 * 11 - L) * scales * np.sqrt(m) * signs[first][None, :]  # m v_0 / sqrt(m) = sqrt(m) v_0
    assert np.all(np.abs(got[:, first] - lead) <= np.abs(lead) * 2.0 ** -8)
    # the normalised product of the storage-rotation oracle is the same weights up to rounding
    w = oracle.dequant(codes, scales, bits, g)
    assert np.allclose(oracle.rotate_rows_inverse(w, m, signs), oracle.materialize_exact(buf, rows, n, bits, g, m, signs, n),
                       atol=1e-15)
