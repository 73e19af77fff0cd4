"""GPU parity of wr_materialize against the oracle (packed module -> bf16 weights in the input basis)."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wr():
    from post_bit_weight_amd import _lib
    return _lib


@pytest.fixture(scope="module")
def ctx(wr):
    return wr.Context(0)


CASES = [  # rows, n_store, bits, group, had_block, n_out
    (37, 1024, 2, 64, 0, 1000),
    (37, 1024, 3, 32, 256, 1000),
    (16, 2560, 2, 64, 512, 2560),
    (5, 10240, 2, 64, 1024, 9728),  # the padded 9728-wide input dim, blocks of 1024
    (4, 776, 3, 8, 0, 770),         # ragged last 512-column segment, 3-bit fields across bytes
    (9, 160, 4, 32, 32, 150),       # blocks below one wave's 64 columns, ragged segment
    (6, 200, 3, 8, 8, 197),
    (3, 4096, 2, 128, 4096, 4096),  # the largest block
    (12, 512, 4, 64, 128, 512),
    (7, 768, 2, 64, 0, 768),
    (8, 1024, 2, 64, 64, 1024),     # one chunk per block: no exchange across lanes
    (6, 2048, 3, 32, 2048, 2040),   # exchanges at lane distances 1, 2, 4, 8 and 16
    (2, 3072, 4, 192, 0, 3072),     # a group spanning three chunks
    (300, 2560, 2, 64, 512, 2560),  # a ragged last workgroup of chunks
]


# "aligned": ld a multiple of 8 (with n_store % 64 == 0 the library takes its chunk kernel);
# "ragged": ld = n_out + 3 (the general kernel)
@pytest.mark.parametrize("layout", ["aligned", "ragged"])
@pytest.mark.parametrize("rows,n,bits,g,m,n_out", CASES)
def test_materialize_matches_oracle(wr, ctx, rows, n, bits, g, m, n_out, layout):
    rng = np.random.default_rng(rows * 7 + n + m)
    L = 2 ** bits - 1
    codes = rng.integers(0, L + 1, size=(rows, n))
    scales = oracle.fp16_rne(rng.uniform(1e-3, 3e-2, size=(rows, n // g)))
    buf = oracle.pack(codes, scales, bits, g)
    signs = rng.choice([-1, 1], size=n).astype(np.int8)
    dbuf = torch.from_numpy(np.ascontiguousarray(buf)).cuda()
    dsig = torch.from_numpy(signs).cuda()
    ld = n_out + 3 if layout == "ragged" else (n_out + 7) // 8 * 8 + 8
    out = torch.zeros(rows, ld, dtype=torch.bfloat16, device="cuda")[:, :n_out]
    wr.wr_materialize(ctx, dbuf, rows, n, bits, g, out, had_block=m, signs=dsig if m else None)
    torch.cuda.synchronize()
    got = out.contiguous().view(torch.int16).cpu().numpy().astype(np.uint16)
    ref = oracle.materialize(buf, rows, n, bits, g, m, signs.astype(np.float64), n_out)
    if m == 0:
        assert np.array_equal(got, ref)
        return
    # fp32 butterflies on the GPU: a bf16 rounding may differ only where the exact weight lies
    # within fp32's error bound of a midpoint.  Each output of a block is a signed sum of the
    # block's m dequantized values over sqrt(m); the scale's rounding, the product and each of
    # the log2(m) butterfly stages add at most 2^-24 of the sum of the terms' magnitudes.
    diff = got != ref
    assert diff.mean() <= 1e-3, diff.mean()
    exact = oracle.materialize_exact(buf, rows, n, bits, g, m, signs.astype(np.float64), n_out)
    codes_d, scales_d = oracle.unpack(buf, rows, n, bits, g)
    absv = np.abs(oracle.dequant(codes_d, scales_d, bits, g)).reshape(rows, n // m, m).sum(axis=2) / np.sqrt(m)
    bound = (np.log2(m) + 4) * 2.0 ** -24 * np.repeat(absv, m, axis=1)[:, :n_out]
    # got must be the bf16 rounding of some value within the bound of the exact weight
    gv, ex = oracle.bf16_bits_to_f64(got[diff]), exact[diff]
    _, e = np.frexp(np.maximum(np.abs(gv), np.abs(ex)))
    assert np.all(np.abs(gv - ex) <= np.ldexp(1.0, e - 9) + bound[diff])


def test_materialize_rejects_bad_arguments(wr, ctx):
    buf = torch.zeros(oracle.packed_bytes(2, 64, 2, 32), dtype=torch.uint8, device="cuda")
    out = torch.zeros(2, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError):
        wr.wr_materialize(ctx, buf[:-1], 2, 64, 2, 32, out)
    with pytest.raises(RuntimeError):
        wr.wr_materialize(ctx, buf, 2, 64, 2, 32, out, had_block=48, signs=torch.ones(64, dtype=torch.int8, device="cuda"))


def _sub_container(buf, rows, n, bits, g, sel):
    """The container of the selected rows alone (codes of those rows, then their scales)."""
    rb, sb = n * bits // 8, 2 * (n // g)
    codes = buf[:rows * rb].reshape(rows, rb)[sel]
    scales = buf[rows * rb:].reshape(rows, sb)[sel]
    return np.concatenate([codes.ravel(), scales.ravel()])


def test_materialize_bench_size_sampled_rows(wr, ctx):
    """The bench launch: 25600 x 2560, 2-bit, group 64, blocks of 512, aligned output; the oracle
    on 48 sampled rows (rows are independent), to the same bar as above."""
    rows, n, bits, g, m = 25600, 2560, 2, 64, 512
    gen = torch.Generator(device="cuda").manual_seed(20261208)
    code_bytes = rows * n * bits // 8
    buf = torch.randint(0, 256, (wr.packed_nbytes(rows, n, bits, g),), dtype=torch.uint8, device="cuda", generator=gen)
    sc = (torch.rand(rows * (n // g), device="cuda", generator=gen) * 0.029 + 1e-3).to(torch.float16)
    buf[code_bytes:] = sc.view(torch.uint8)
    signs = (torch.randint(0, 2, (n,), device="cuda", generator=gen) * 2 - 1).to(torch.int8)
    out = torch.empty(rows, n, dtype=torch.bfloat16, device="cuda")
    wr.wr_materialize(ctx, buf, rows, n, bits, g, out, had_block=m, signs=signs)
    torch.cuda.synchronize()
    sel = np.sort(np.r_[0, rows - 1, np.random.default_rng(9).choice(np.arange(1, rows - 1), 46, replace=False)])
    sub = _sub_container(buf.cpu().numpy(), rows, n, bits, g, sel)
    sg = signs.cpu().numpy().astype(np.float64)
    ref = oracle.materialize(sub, sel.size, n, bits, g, m, sg, n)
    got = out[torch.as_tensor(sel, device="cuda")].view(torch.int16).cpu().numpy().astype(np.uint16)
    diff = got != ref
    assert diff.mean() <= 1e-3, diff.mean()
    exact = oracle.materialize_exact(sub, sel.size, n, bits, g, m, sg, n)
    codes_d, scales_d = oracle.unpack(sub, sel.size, n, bits, g)
    absv = np.abs(oracle.dequant(codes_d, scales_d, bits, g)).reshape(sel.size, n // m, m).sum(axis=2) / np.sqrt(m)
    bound = (np.log2(m) + 4) * 2.0 ** -24 * np.repeat(absv, m, axis=1)
    gv, ex = oracle.bf16_bits_to_f64(got[diff]), exact[diff]
    _, e = np.frexp(np.maximum(np.abs(gv), np.abs(ex)))
    assert np.all(np.abs(gv - ex) <= np.ldexp(1.0, e - 9) + bound[diff])
