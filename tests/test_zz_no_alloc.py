"""The allocation-free H accumulation against the workspace one, through the C ABI.

Two calls in a row on one GPU (they share its static scratch), the second with a smaller input:
bf16 calibration rows whose split partials exceed the static scratch (the call runs in row
slices, so its fp32 split sums differ from the workspace call's: both must agree within the
1e-5 relative Frobenius bar of H), then fp32 rows whose workspace need fits the static scratch
(the same launches as the workspace call: bit-identical)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _s_pair(wr, ctx, X, zero_first=True):
    n = X.shape[1]
    S_ws = torch.full((n, n), float("nan"), dtype=torch.float64, device="cuda")
    S_na = torch.full((n, n), float("nan"), dtype=torch.float64, device="cuda")
    wr.wr_hessian_accumulate(ctx, X, S_ws, zero=zero_first)
    wr.wr_hessian_accumulate_noalloc(ctx, X, S_na, zero=zero_first)
    torch.cuda.synchronize()
    lo = torch.tril(torch.ones(n, n, dtype=torch.bool, device="cuda"))
    return S_ws[lo].cpu().numpy(), S_na[lo].cpu().numpy()


def test_noalloc_matches_the_workspace_entry_point_twice():
    from post_bit_weight_amd import _lib as wr
    from post_bit_weight_amd import synth
    ctx = wr.Context(0)
    # first call: 40960 x 2560 bf16 -- the workspace call's partials (5 splits x 55 tiles x 256 KiB)
    # exceed the static scratch, so the allocation-free call runs row slices of 4 splits
    n = 2560
    need = wr.wr_workspace_bytes(wr.WR_OP_HESSIAN, 40960, n)
    assert need > wr.WR_STATIC_SCRATCH_BYTES
    X = synth.SpectralSource(n, seed=71, device="cuda", outlier_frac=0.01).chunk(0, 40960)
    a, b = _s_pair(wr, ctx, X)
    assert np.isfinite(a).all() and np.isfinite(b).all()
    rel = np.linalg.norm(a - b) / np.linalg.norm(a)
    print(f"bf16 40960 x 2560: relative difference {rel:.2e}")
    assert rel <= 1e-5
    # second call, smaller: 3000 x 512 fp32 (ragged last stage), workspace need within the scratch:
    # the same launches, so the same bits
    n = 512
    assert wr.wr_workspace_bytes(wr.WR_OP_HESSIAN, 3000, n) <= wr.WR_STATIC_SCRATCH_BYTES
    X = synth.SpectralSource(n, seed=72, n_outliers=5).chunk(0, 3000, dtype=torch.float32).cuda()
    a, b = _s_pair(wr, ctx, X)
    assert np.array_equal(a, b)
    # the oracle's definition on the same rows (fp64 X^T X of the fp32 inputs)
    Xh = X.double().cpu().numpy()
    ref = (Xh.T @ Xh)[np.tril_indices(n)]
    assert np.linalg.norm(b - ref) / np.linalg.norm(ref) <= 1e-5


def test_noalloc_argument_errors_launch_nothing():
    from post_bit_weight_amd import _lib as wr
    lib = wr.load()
    assert lib.wr_hessian_accumulate_noalloc(None, None, 1, 0, 8, 8, None, 0) == wr.WR_EINVAL
    ctx = wr.Context(0)
    S = torch.zeros(8, 8, dtype=torch.float64, device="cuda")
    # n not a multiple of 8
    assert lib.wr_hessian_accumulate_noalloc(ctx.handle, None, 1, 0, 12, 12, S.data_ptr(), 1) == wr.WR_EINVAL
    # fp32 input too wide for 512 rows of parts in the static scratch: refused before any launch
    # (S and X have their full sizes, so nothing could go out of bounds even if a launch happened)
    n = 21848
    S_big = torch.full((n, n), float("nan"), dtype=torch.float64, device="cuda")
    X = torch.zeros(1, n, dtype=torch.float32, device="cuda")
    st = lib.wr_hessian_accumulate_noalloc(ctx.handle, X.data_ptr(), wr.WR_F32, 1, n, n, S_big.data_ptr(), 1)
    torch.cuda.synchronize()
    assert st == wr.WR_ESCRATCH
    assert b"static scratch" in lib.wr_strerror(st)
    assert torch.isnan(S_big[::997, ::991]).all()          # WR_H_ZERO was not applied: nothing ran
    del S_big
