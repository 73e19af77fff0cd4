"""ctypes binding of ``libwringer.so`` -- argument marshalling only.

Every function here has the name of the C entry point it calls, takes torch
tensors that already live on the GPU, checks their dtype / device / layout and
passes raw pointers plus the current HIP stream.  No arithmetic of the method
happens in Python; if the shared library is missing, importing any function
raises instead of falling back to anything else.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwringer.so")

WR_OK, WR_EINVAL, WR_EWORKSPACE, WR_EHIP, WR_EUNSUPPORTED, WR_ESCRATCH = 0, 1, 2, 3, 4, 5
WR_STATIC_SCRATCH_BYTES = 64 << 20
WR_F32, WR_BF16 = 0, 1
(WR_OP_HESSIAN, WR_OP_GPTQ, WR_OP_WRING, WR_OP_ROTATE, WR_OP_FINALIZE, WR_OP_WRING_GPTQ, WR_OP_TRELLIS,
 WR_OP_GEMV, WR_OP_STATS) = range(9)
WR_H_ZERO = 1
WR_ROT_ROWS, WR_ROT_ROWS_INVERSE, WR_ROT_SYM = 0, 1, 2
WR_RECODE_NEAREST = 1
WR_RECODE_GPTQ = 2
WR_RECODE_SEARCH = 4

EXPORTED = (
    "wr_create", "wr_destroy", "wr_workspace_bytes", "wr_set_workspace",
    "wr_hessian_accumulate", "wr_hessian_accumulate_noalloc", "wr_hessian_finalize", "wr_hadamard_rotate",
    "wr_gptq_sweep", "wr_wring_solve", "wr_pack", "wr_unpack", "wr_materialize", "wr_trellis_quantize",
    "wr_packed_gemv", "wr_set_scale_trace", "wr_wring_target", "wr_quant_stats", "wr_strerror",
)


class WringerError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {_strerror(status)} (status {status})")
        self.status = status


_lib = None


def _open(path):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with post_bit_weight_amd/csrc/build.py")
    return ctypes.CDLL(path)


def load():
    """Load the HIP library once; raise loudly if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    lib = _open(LIB_PATH)
    c = ctypes
    P, I, I64, F, SZ = c.c_void_p, c.c_int, c.c_int64, c.c_float, c.c_size_t
    sig = {
        "wr_create": (I, [c.POINTER(P), I, P]),
        "wr_destroy": (I, [P]),
        "wr_workspace_bytes": (SZ, [I, I64, I64, c.c_int32, c.c_int32, c.c_int32]),
        "wr_set_workspace": (I, [P, P, SZ]),
        "wr_hessian_accumulate": (I, [P, P, I, I64, I64, I64, P, I]),
        "wr_hessian_accumulate_noalloc": (I, [P, P, I, I64, I64, I64, P, I]),
        "wr_hessian_finalize": (I, [P, P, I64, I64, F, I64, P, I64, P, c.c_int32, P]),
        "wr_hadamard_rotate": (I, [P, P, I64, I64, I64, c.c_int32, P, I]),
        "wr_gptq_sweep": (I, [P, P, I, I64, I64, I64, P, I64, P, c.c_int32, c.c_int32, P, P, P]),
        "wr_wring_solve": (I, [P, P, I, I64, P, P, c.c_int32, F, I, P, I64, I64, I64, P, c.c_int32, F, I, P, P, P]),
        "wr_pack": (I, [P, P, P, I64, I64, c.c_int32, c.c_int32, P, SZ]),
        "wr_unpack": (I, [P, P, SZ, I64, I64, c.c_int32, c.c_int32, P, P, P]),
        "wr_materialize": (I, [P, P, SZ, I64, I64, c.c_int32, c.c_int32, c.c_int32, P, I64, P, I64]),
        "wr_trellis_quantize": (I, [P, P, I64, I64, I64, c.c_int32, c.c_int32, P, c.c_int32, P, I64, P, I64, P]),
        "wr_packed_gemv": (I, [P, P, SZ, I64, I64, c.c_int32, c.c_int32, c.c_int32, P, P, I64, I64, c.c_int32, P,
                               I64]),
        "wr_set_scale_trace": (I, [P, P, I64]),
        "wr_wring_target": (I, [P, P, I, I64, P, P, c.c_int32, F, I, I64, I64, P, c.c_int32, P, P, P, P]),
        "wr_quant_stats": (I, [P, P, I64, P, P, P, I64, I64, c.c_int32, P, P, P]),
        "wr_strerror": (c.c_char_p, [I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _strerror(status):
    try:
        return load().wr_strerror(status).decode()
    except Exception:  # pragma: no cover - only when the library itself is missing
        return "unknown"


def _check(fn, status):
    if status != WR_OK:
        raise WringerError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtypes):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def _rowmajor(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D row-major tensor")
    return t.stride(0)


def _wdtype(t):
    return WR_BF16 if t.dtype == torch.bfloat16 else WR_F32


FLOATS = (torch.float32, torch.bfloat16)


class Context:
    """One library context bound to a device and a HIP stream, plus its workspace tensor."""

    def __init__(self, device=0, stream=None):
        lib = load()
        self.device = torch.device("cuda", device) if isinstance(device, int) else torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        h = ctypes.c_void_p()
        _check("wr_create", lib.wr_create(ctypes.byref(h), self.device.index or 0, ctypes.c_void_p(self.stream.cuda_stream)))
        self.handle = h
        self.workspace = None

    def ensure_workspace(self, nbytes):
        if self.workspace is None or self.workspace.numel() < nbytes:
            self.workspace = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=self.device)
            _check("wr_set_workspace", load().wr_set_workspace(self.handle, _ptr(self.workspace), self.workspace.numel()))

    def close(self):
        if self.handle:
            load().wr_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def wr_workspace_bytes(op, rows, n, group=0, rank=0, lazy_batch=0):
    return int(load().wr_workspace_bytes(op, rows, n, group, rank, lazy_batch))


def wr_hessian_accumulate(ctx, X, S, zero=False):
    """S (n x n fp64) += X^T X for the rows of X (bf16 or fp32)."""
    _dev(X, "X", FLOATS)
    _dev(S, "S", (torch.float64,))
    rows, n = X.shape
    ldx = _rowmajor(X, "X")
    if tuple(S.shape) != (n, n) or not S.is_contiguous():
        raise ValueError("S must be a contiguous n x n fp64 tensor")
    ctx.ensure_workspace(wr_workspace_bytes(WR_OP_HESSIAN, rows, n))
    _check("wr_hessian_accumulate", load().wr_hessian_accumulate(
        ctx.handle, _ptr(X), _wdtype(X), rows, n, ldx, _ptr(S), WR_H_ZERO if zero else 0))


def wr_hessian_accumulate_noalloc(ctx, X, S, zero=False):
    """As wr_hessian_accumulate, without the registered workspace (the library's static scratch)."""
    _dev(X, "X", FLOATS)
    _dev(S, "S", (torch.float64,))
    rows, n = X.shape
    ldx = _rowmajor(X, "X")
    if tuple(S.shape) != (n, n) or not S.is_contiguous():
        raise ValueError("S must be a contiguous n x n fp64 tensor")
    _check("wr_hessian_accumulate_noalloc", load().wr_hessian_accumulate_noalloc(
        ctx.handle, _ptr(X), _wdtype(X), rows, n, ldx, _ptr(S), WR_H_ZERO if zero else 0))


def wr_hessian_finalize(ctx, S, total_rows, damp_frac, H, delta=None, had_block=0, signs=None):
    """H (n_store x n_store fp32) = R pad(S / total_rows) R^T + delta I (R = I when had_block is 0)."""
    _dev(S, "S", (torch.float64,))
    _dev(H, "H", (torch.float32,))
    _dev(delta, "delta", (torch.float32,))
    _dev(signs, "signs", (torch.int8,))
    n = S.shape[0]
    ldh = _rowmajor(H, "H")
    if had_block:
        if signs is None or signs.numel() != H.shape[0] or not signs.is_contiguous():
            raise ValueError("signs must hold n_store contiguous int8 values")
        ctx.ensure_workspace(wr_workspace_bytes(WR_OP_FINALIZE, 0, H.shape[0]))
    else:
        ctx.ensure_workspace(256)
    _check("wr_hessian_finalize", load().wr_hessian_finalize(
        ctx.handle, _ptr(S), n, int(total_rows), float(damp_frac), H.shape[0], _ptr(H), ldh, _ptr(delta),
        int(had_block or 0), _ptr(signs)))


def wr_hadamard_rotate(ctx, M, had_block, signs, mode=WR_ROT_ROWS):
    _dev(M, "M", (torch.float32,))
    _dev(signs, "signs", (torch.int8,))
    rows, n = M.shape
    ld = _rowmajor(M, "M")
    if signs.numel() != n or not signs.is_contiguous():
        raise ValueError("signs must hold n contiguous int8 values")
    _check("wr_hadamard_rotate", load().wr_hadamard_rotate(ctx.handle, _ptr(M), rows, n, ld, int(had_block), _ptr(signs), mode))


def wr_gptq_sweep(ctx, W, H, bits, group, lazy_batch, codes, scales, dev_info):
    _dev(W, "W", FLOATS)
    _dev(H, "H", (torch.float32,))
    _dev(bits, "bits", (torch.uint8,))
    _dev(codes, "codes", (torch.uint8,))
    _dev(scales, "scales", (torch.float16, torch.int16, torch.uint16))
    _dev(dev_info, "dev_info", (torch.int32,))
    rows, n = W.shape
    ldw = _rowmajor(W, "W")
    ldh = _rowmajor(H, "H")
    if tuple(codes.shape) != (rows, n) or not codes.is_contiguous():
        raise ValueError("codes must be a contiguous rows x n uint8 tensor")
    if tuple(scales.shape) != (rows, n // group) or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous rows x n/group fp16 tensor")
    if bits.numel() != rows:
        raise ValueError("bits must hold one value per row")
    ctx.ensure_workspace(wr_workspace_bytes(WR_OP_GPTQ, rows, n, group, 0, lazy_batch))
    _check("wr_gptq_sweep", load().wr_gptq_sweep(
        ctx.handle, _ptr(W), _wdtype(W), rows, n, ldw, _ptr(H), ldh, _ptr(bits), int(group), int(lazy_batch),
        _ptr(codes), _ptr(scales), _ptr(dev_info)))


def wr_wring_solve(ctx, H, bits, group, lam, codes, scales, dev_info, target=None, B=None, A=None, alpha=0.0,
                   recode=False):
    """recode: False (joint scales only), True or "nearest" (WR_RECODE_NEAREST), "gptq" (WR_RECODE_GPTQ),
    "search" (WR_RECODE_SEARCH: searched block scales, no joint solve; H may be None)."""
    if recode not in (False, True, "nearest", "gptq", "search"):
        raise ValueError("recode must be False, True, 'nearest', 'gptq' or 'search'")
    flags = {"gptq": WR_RECODE_GPTQ, "search": WR_RECODE_SEARCH}.get(recode, WR_RECODE_NEAREST if recode else 0)
    _dev(target, "target", FLOATS)
    _dev(B, "B", FLOATS)
    _dev(A, "A", FLOATS)
    _dev(H, "H", (torch.float32,))
    _dev(bits, "bits", (torch.uint8,))
    _dev(codes, "codes", (torch.uint8,))
    _dev(scales, "scales", (torch.float16, torch.int16, torch.uint16))
    _dev(dev_info, "dev_info", (torch.int32,))
    rows, n = codes.shape
    ldh = _rowmajor(H, "H") if H is not None else 0
    ldt = _rowmajor(target, "target") if target is not None else 0
    rank = 0
    ab_dtype = WR_F32
    if B is not None:
        if A is None or B.dtype != A.dtype or not B.is_contiguous() or not A.is_contiguous():
            raise ValueError("B and A must be contiguous tensors of one dtype")
        rank = A.shape[0]
        if tuple(B.shape) != (rows, rank) or tuple(A.shape) != (rank, n):
            raise ValueError("B must be rows x r and A r x n")
        ab_dtype = _wdtype(A)
    op = WR_OP_WRING_GPTQ if flags == WR_RECODE_GPTQ else WR_OP_WRING
    ctx.ensure_workspace(wr_workspace_bytes(op, rows, n, group, rank, 0))
    _check("wr_wring_solve", load().wr_wring_solve(
        ctx.handle, _ptr(target), _wdtype(target) if target is not None else WR_F32, ldt, _ptr(B), _ptr(A), rank,
        float(alpha), ab_dtype, _ptr(H), ldh, rows, n, _ptr(bits), int(group), float(lam),
        flags, _ptr(codes), _ptr(scales), _ptr(dev_info)))


def wr_materialize(ctx, buf, rows, n_store, bits, group, out, had_block=0, signs=None):
    """bf16 weights (out: rows x n_out bf16, n_out <= n_store) from one packed module."""
    _dev(buf, "buf", (torch.uint8,))
    _dev(out, "out", (torch.bfloat16, torch.int16, torch.uint16))
    _dev(signs, "signs", (torch.int8,))
    if out.dim() != 2 or out.shape[0] != rows:
        raise ValueError("out must be rows x n_out")
    ldo = _rowmajor(out, "out")
    _check("wr_materialize", load().wr_materialize(ctx.handle, _ptr(buf), buf.numel(), rows, n_store, int(bits),
                                                   int(group), int(had_block), _ptr(signs), out.shape[1], _ptr(out),
                                                   ldo))


def packed_nbytes(rows, n, bits, group):
    return rows * n * bits // 8 + 2 * rows * (n // group)


def wr_pack(ctx, codes, scales, bits, group, out):
    _dev(codes, "codes", (torch.uint8,))
    _dev(scales, "scales", (torch.float16, torch.int16, torch.uint16))
    _dev(out, "out", (torch.uint8,))
    rows, n = codes.shape
    if not codes.is_contiguous() or not scales.is_contiguous() or not out.is_contiguous():
        raise ValueError("codes, scales and out must be contiguous")
    _check("wr_pack", load().wr_pack(ctx.handle, _ptr(codes), _ptr(scales), rows, n, int(bits), int(group), _ptr(out),
                                     out.numel()))


def wr_unpack(ctx, buf, rows, n, bits, group, codes=None, scales=None, dequant=None):
    _dev(buf, "buf", (torch.uint8,))
    _dev(codes, "codes", (torch.uint8,))
    _dev(scales, "scales", (torch.float16, torch.int16, torch.uint16))
    _dev(dequant, "dequant", (torch.bfloat16,))
    _check("wr_unpack", load().wr_unpack(ctx.handle, _ptr(buf), buf.numel(), rows, n, int(bits), int(group),
                                         _ptr(codes), _ptr(scales), _ptr(dequant)))


def wr_trellis_quantize(ctx, T, log2_states, values, codes, recon=None, cost=None, start_state=0):
    """Viterbi search of a shift-register trellis for each row of T (rows x n fp32).

    values: S x 2 x C fp32 device tensor (the coset of each branch); codes: rows x n uint8;
    recon: optional rows x n fp32; cost: optional rows fp64."""
    _dev(T, "T", (torch.float32,))
    _dev(values, "values", (torch.float32,))
    _dev(codes, "codes", (torch.uint8,))
    _dev(recon, "recon", (torch.float32,))
    _dev(cost, "cost", (torch.float64,))
    rows, n = T.shape
    S = 1 << int(log2_states)
    if values.dim() != 3 or values.shape[0] != S or values.shape[1] != 2 or not values.is_contiguous():
        raise ValueError("values must be a contiguous S x 2 x C tensor")
    if tuple(codes.shape) != (rows, n) or (recon is not None and tuple(recon.shape) != (rows, n)):
        raise ValueError("codes and recon must be rows x n")
    if cost is not None and (cost.numel() != rows or not cost.is_contiguous()):
        raise ValueError("cost must hold one value per row")
    ctx.ensure_workspace(wr_workspace_bytes(WR_OP_TRELLIS, rows, n, S))
    _check("wr_trellis_quantize", load().wr_trellis_quantize(
        ctx.handle, _ptr(T), _rowmajor(T, "T"), rows, n, int(log2_states), values.shape[2], _ptr(values),
        int(start_state), _ptr(codes), _rowmajor(codes, "codes"), _ptr(recon),
        _rowmajor(recon, "recon") if recon is not None else 0, _ptr(cost)))


def wr_packed_gemv(ctx, buf, rows, n_store, bits, group, x, y, had_block=0, signs=None):
    """y (batch x rows fp32) = the packed module's weights in the input basis times each row of x
    (batch x n_in fp32, n_in <= n_store)."""
    _dev(buf, "buf", (torch.uint8,))
    _dev(x, "x", (torch.float32,))
    _dev(y, "y", (torch.float32,))
    _dev(signs, "signs", (torch.int8,))
    if x.dim() != 2 or y.dim() != 2 or y.shape[0] != x.shape[0] or y.shape[1] != rows:
        raise ValueError("x must be batch x n_in and y batch x rows")
    batch = x.shape[0]
    ctx.ensure_workspace(wr_workspace_bytes(WR_OP_GEMV, batch, n_store))
    _check("wr_packed_gemv", load().wr_packed_gemv(ctx.handle, _ptr(buf), buf.numel(), rows, n_store, int(bits),
                                                   int(group), int(had_block), _ptr(signs), _ptr(x), x.shape[1],
                                                   _rowmajor(x, "x"), batch, _ptr(y), _rowmajor(y, "y")))


def wr_set_scale_trace(ctx, raw=None):
    """Later joint solves on ctx also write their unprojected scales (fp32) into raw; None stops it."""
    _dev(raw, "raw", (torch.float32,))
    if raw is not None and not raw.is_contiguous():
        raise ValueError("raw must be contiguous")
    _check("wr_set_scale_trace", load().wr_set_scale_trace(ctx.handle, _ptr(raw), raw.numel() if raw is not None else 0))
    ctx.scale_trace = raw


def wr_wring_target(ctx, bits, group, T_out, dev_info, target=None, codes=None, scales=None, B=None, A=None,
                    alpha=0.0):
    """T_out (rows x n fp32) = target or dequant(codes, scales), plus (alpha / r) B A."""
    _dev(target, "target", FLOATS)
    _dev(B, "B", FLOATS)
    _dev(A, "A", FLOATS)
    _dev(bits, "bits", (torch.uint8,))
    _dev(codes, "codes", (torch.uint8,))
    _dev(scales, "scales", (torch.float16, torch.int16, torch.uint16))
    _dev(T_out, "T_out", (torch.float32,))
    _dev(dev_info, "dev_info", (torch.int32,))
    rows, n = T_out.shape
    if not T_out.is_contiguous():
        raise ValueError("T_out must be contiguous")
    ldt = _rowmajor(target, "target") if target is not None else 0
    rank, ab_dtype = 0, WR_F32
    if B is not None:
        if A is None or B.dtype != A.dtype or not B.is_contiguous() or not A.is_contiguous():
            raise ValueError("B and A must be contiguous tensors of one dtype")
        rank = A.shape[0]
        if tuple(B.shape) != (rows, rank) or tuple(A.shape) != (rank, n):
            raise ValueError("B must be rows x r and A r x n")
        ab_dtype = _wdtype(A)
    ctx.ensure_workspace(wr_workspace_bytes(WR_OP_WRING, rows, n, group, rank, 0))
    _check("wr_wring_target", load().wr_wring_target(
        ctx.handle, _ptr(target), _wdtype(target) if target is not None else WR_F32, ldt, _ptr(B), _ptr(A), rank,
        float(alpha), ab_dtype, rows, n, _ptr(bits), int(group), _ptr(codes), _ptr(scales), _ptr(T_out),
        _ptr(dev_info)))


def wr_quant_stats(ctx, codes, scales, bits, group, out, T=None, codes_ref=None, scales_raw=None):
    """out (4 fp64, device): [sum (t - dequant)^2, sum t^2, codes differing from codes_ref,
    weights whose bf16 rounding moves between the fp16 and the unprojected scales]."""
    _dev(T, "T", (torch.float32,))
    _dev(codes, "codes", (torch.uint8,))
    _dev(codes_ref, "codes_ref", (torch.uint8,))
    _dev(scales, "scales", (torch.float16, torch.int16, torch.uint16))
    _dev(scales_raw, "scales_raw", (torch.float32,))
    _dev(bits, "bits", (torch.uint8,))
    _dev(out, "out", (torch.float64,))
    rows, n = codes.shape
    for t, name in ((codes, "codes"), (scales, "scales"), (codes_ref, "codes_ref"), (scales_raw, "scales_raw")):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if out.numel() < 4:
        raise ValueError("out must hold 4 values")
    ctx.ensure_workspace(wr_workspace_bytes(WR_OP_STATS, rows, n))
    _check("wr_quant_stats", load().wr_quant_stats(
        ctx.handle, _ptr(T), _rowmajor(T, "T") if T is not None else 0, _ptr(codes), _ptr(scales), _ptr(bits), rows, n,
        int(group), _ptr(codes_ref), _ptr(scales_raw), _ptr(out)))
