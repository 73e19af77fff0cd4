"""GPU parity of wr_packed_gemv (packed module times input vectors) against the oracle.

The GPU forms x' = R x_pad and the products in fp32; each output may differ from the oracle's
fp64 result by fp32's error bound relative to its sum of term magnitudes:
  |dy| <= (64 + 4 L) 2^-24 sum_j |w_j| (|x'_j| + A_j),
where A_j = (log2 m + 2) times the block's sum of |x| over sqrt(m) accounts for the rounding of
x' itself, 64 covers the sums of 32 products, of the chunks and of the 16 lanes of a row, and
4 L the cancellation in 2 sum c x' - L sum x' (the level 2c - L split into two sums).
"""
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


def _bound(buf, rows, n, n_in, bits, g, m, signs, X):
    L = 2 ** bits - 1
    codes, scales = oracle.unpack(buf, rows, n, bits, g)
    Wq = np.abs(oracle.dequant(codes, scales, bits, g))
    Xp = np.zeros((X.shape[0], n))
    Xp[:, :n_in] = X
    xr = np.abs(oracle.rotate_rows(Xp, m, signs)) if m else np.abs(Xp)
    if m:
        A = (np.log2(m) + 2) * np.repeat(np.abs(Xp).reshape(X.shape[0], n // m, m).sum(axis=2), m, axis=1) / np.sqrt(m)
    else:
        A = np.zeros_like(Xp)
    return (64 + 4 * L) * 2.0 ** -24 * ((xr + A) @ Wq.T)


CASES = [  # rows, n_store, n_in, bits, group, had_block, batch
    (37, 1024, 1000, 2, 64, 0, 1),
    (37, 1024, 1000, 3, 32, 256, 3),
    (16, 2560, 2560, 2, 64, 512, 1),
    (5, 10240, 9728, 2, 64, 1024, 8),
    (300, 2560, 2560, 4, 128, 512, 4),
    (3, 4096, 4096, 2, 64, 4096, 2),
    (9, 96, 90, 2, 32, 32, 1),
    (40, 2560, 2560, 3, 64, 512, 5),
    (20, 4096, 4096, 2, 64, 256, 6),  # x' too large for LDS: rotation kernel + product from global memory
    (33, 512, 500, 2, 64, 64, 2),     # blocks of one wave's 64 lanes, one element each
    (7, 1024, 1024, 3, 32, 128, 1),
]


@pytest.mark.parametrize("rows,n,n_in,bits,g,m,batch", CASES)
def test_packed_gemv_matches_oracle(wr, ctx, rows, n, n_in, bits, g, m, batch):
    rng = np.random.default_rng(rows + n + batch)
    L = 2 ** bits - 1
    codes = rng.integers(0, L + 1, size=(rows, n))
    scales = oracle.fp16_rne(rng.uniform(1e-3, 3e-2, size=(rows, n // g)))
    buf = oracle.pack(codes, scales, bits, g)
    signs = rng.choice([-1, 1], size=n).astype(np.int8)
    X = rng.normal(size=(batch, n_in)).astype(np.float32)
    x_t = torch.zeros(batch, n_in + 5, dtype=torch.float32, device="cuda")[:, :n_in]  # ld > n_in
    x_t.copy_(torch.from_numpy(X))
    y = torch.full((batch, rows), float("nan"), dtype=torch.float32, device="cuda")
    wr.wr_packed_gemv(ctx, torch.from_numpy(buf).cuda(), rows, n, bits, g, x_t, y, had_block=m,
                      signs=torch.from_numpy(signs).cuda() if m else None)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    ref = oracle.packed_gemv(buf, rows, n, bits, g, m, signs.astype(np.float64), X.astype(np.float64))
    bound = _bound(buf, rows, n, n_in, bits, g, m, signs.astype(np.float64), X.astype(np.float64))
    assert np.all(np.abs(got - ref) <= bound), np.max(np.abs(got - ref) / bound)


def test_packed_gemv_bench_size(wr, ctx):
    """The bench launch: 25600 x 2560, 2-bit, group 64, blocks of 512, one vector; the oracle on 64
    sampled rows."""
    rows, n, bits, g, m = 25600, 2560, 2, 64, 512
    gen = torch.Generator(device="cuda").manual_seed(20261240)
    code_bytes = rows * n * bits // 8
    buf = torch.randint(0, 256, (wr.packed_nbytes(rows, n, bits, g),), dtype=torch.uint8, device="cuda", generator=gen)
    sc = (torch.rand(rows * (n // g), device="cuda", generator=gen) * 0.029 + 1e-3).to(torch.float16)
    buf[code_bytes:] = sc.view(torch.uint8)
    signs = (torch.randint(0, 2, (n,), device="cuda", generator=gen) * 2 - 1).to(torch.int8)
    x = torch.randn(1, n, device="cuda", generator=gen)
    y = torch.empty(1, rows, dtype=torch.float32, device="cuda")
    wr.wr_packed_gemv(ctx, buf, rows, n, bits, g, x, y, had_block=m, signs=signs)
    torch.cuda.synchronize()
    sel = np.sort(np.r_[0, rows - 1, np.random.default_rng(13).choice(np.arange(1, rows - 1), 62, replace=False)])
    rb, sb = n * bits // 8, 2 * (n // g)
    hb = buf.cpu().numpy()
    sub = np.concatenate([hb[:rows * rb].reshape(rows, rb)[sel].ravel(), hb[rows * rb:].reshape(rows, sb)[sel].ravel()])
    X = x.cpu().numpy().astype(np.float64)
    sg = signs.cpu().numpy().astype(np.float64)
    ref = oracle.packed_gemv(sub, sel.size, n, bits, g, m, sg, X)
    bound = _bound(sub, sel.size, n, n, bits, g, m, sg, X)
    got = y[:, torch.as_tensor(sel, device="cuda")].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= bound)


def test_packed_gemv_rejects_bad_arguments(wr, ctx):
    buf = torch.zeros(oracle.packed_bytes(4, 64, 2, 32), dtype=torch.uint8, device="cuda")
    x = torch.zeros(1, 64, dtype=torch.float32, device="cuda")
    y = torch.zeros(1, 4, dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError):  # wrong container size
        wr.wr_packed_gemv(ctx, buf[:-2], 4, 64, 2, 32, x, y)
    with pytest.raises(RuntimeError):  # group not a multiple of 32
        wr.wr_packed_gemv(ctx, torch.zeros(oracle.packed_bytes(4, 64, 2, 16), dtype=torch.uint8, device="cuda"),
                          4, 64, 2, 16, x, y)
