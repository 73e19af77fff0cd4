"""Sequence the library calls that quantize one linear layer (or several layers sharing H).

Order (Wringer model cards, "Recipe"; Wringer news article, second paragraph):
H accumulation and damping -> optional Hadamard rotation -> GPTQ codes and
scales -> joint scales against the weights -> wring against
W_hat + (alpha / r) B A (nearest-point codes, joint scales) -> packing.
Every step runs in libwringer.so; torch only allocates device memory and pads
the weights into the stored (rotated) dimension.
"""

import torch

from . import _lib as wr


def accumulate_hessian(ctx, chunks, n, S=None):
    """S (n x n fp64) = sum over chunks of X^T X; returns (S, total_rows)."""
    if S is None:
        S = torch.empty(n, n, dtype=torch.float64, device=ctx.device)
    total = 0
    first = True
    for X in chunks:
        wr.wr_hessian_accumulate(ctx, X, S, zero=first)
        first = False
        total += X.shape[0]
    if first:
        wr.wr_hessian_accumulate(ctx, torch.empty(0, n, dtype=torch.bfloat16, device=ctx.device), S, zero=True)
    return S, total


def finalize_hessian(ctx, S, total_rows, damp_frac, n_store, had_block=None, signs=None):
    H = torch.empty(n_store, n_store, dtype=torch.float32, device=ctx.device)
    delta = torch.empty(1, dtype=torch.float32, device=ctx.device)
    wr.wr_hessian_finalize(ctx, S, total_rows, damp_frac, H, delta, had_block or 0, signs)
    return H, delta


def prepare_weights(ctx, W, n_store, had_block=None, signs=None):
    """The weights in the stored basis: zero-padded to n_store and rotated when had_block is set."""
    rows, n0 = W.shape
    if not had_block and n_store == n0:
        return W
    Wp = torch.zeros(rows, n_store, dtype=torch.float32, device=ctx.device)
    Wp[:, :n0] = W
    if had_block:
        wr.wr_hadamard_rotate(ctx, Wp, had_block, signs, wr.WR_ROT_ROWS)
    return Wp


def quantize(ctx, Wst, H, bits, group, lam=0.01, B=None, A=None, alpha=None, lazy_batch=128, keep_stages=False,
             finisher="nearest", adapters=None):
    """GPTQ sweep, joint scales, wring.  bits: int or a per-row uint8 tensor.  finisher: "nearest"
    (nearest-point codes on the current scales) or "gptq" (a GPTQ sweep of the watered target).
    adapters: a sequence of (B, A) pairs for several fill-and-wring rounds, each wring starting
    from the previous one's codes and scales (instead of B and A).  Returns a dict of tensors."""
    if finisher not in ("nearest", "gptq"):
        raise ValueError("finisher must be 'nearest' or 'gptq'")
    if adapters is not None and B is not None:
        raise ValueError("pass either B and A or adapters")
    if adapters is None:
        adapters = [] if B is None else [(B, A)]
    rows, n = Wst.shape
    if isinstance(bits, int):
        bits_t = torch.full((rows,), bits, dtype=torch.uint8, device=ctx.device)
    else:
        bits_t = bits
    codes = torch.empty(rows, n, dtype=torch.uint8, device=ctx.device)
    scales = torch.empty(rows, n // group, dtype=torch.float16, device=ctx.device)
    info = torch.zeros(2 + max(1, len(adapters)), dtype=torch.int32, device=ctx.device)
    out = {}
    wr.wr_gptq_sweep(ctx, Wst, H, bits_t, group, lazy_batch, codes, scales, info[0:1])
    if keep_stages:
        out["gptq_codes"], out["gptq_scales"] = codes.clone(), scales.clone()
    wr.wr_wring_solve(ctx, H, bits_t, group, lam, codes, scales, info[1:2], target=Wst)
    if keep_stages:
        out["joint_scales"] = scales.clone()
    for k, (Bk, Ak) in enumerate(adapters):
        wr.wr_wring_solve(ctx, H, bits_t, group, lam, codes, scales, info[2 + k:3 + k], B=Bk, A=Ak,
                          alpha=alpha if alpha is not None else Ak.shape[0],
                          recode="gptq" if finisher == "gptq" else True)
        if keep_stages and k + 1 < len(adapters):
            out[f"round{k + 1}_codes"], out[f"round{k + 1}_scales"] = codes.clone(), scales.clone()
    out.update(codes=codes, scales=scales, dev_info=info, bits=bits_t)
    return out


def pack(ctx, codes, scales, bits, group):
    rows, n = codes.shape
    buf = torch.empty(wr.packed_nbytes(rows, n, bits, group), dtype=torch.uint8, device=ctx.device)
    wr.wr_pack(ctx, codes, scales, bits, group, buf)
    return buf


def solve_module(ctx, W, chunks, bits, group, damp_frac=0.01, lam=0.01, B=None, A=None, alpha=None,
                 had_block=None, signs=None, n_store=None, lazy_batch=128, keep_stages=False):
    """The whole solve for one module W (rows x n0) with calibration chunks (each N_k x n0)."""
    rows, n0 = W.shape
    n = n_store or n0
    S, total = accumulate_hessian(ctx, chunks, n0)
    H, delta = finalize_hessian(ctx, S, total, damp_frac, n, had_block, signs)
    Wst = prepare_weights(ctx, W, n, had_block, signs)
    out = quantize(ctx, Wst, H, bits, group, lam, B, A, alpha, lazy_batch, keep_stages)
    if isinstance(bits, int):
        out["packed"] = pack(ctx, out["codes"], out["scales"], bits, group)
    out.update(H=H, delta=delta, S=S, W=Wst)
    return out


def solve_group(ctx, modules, H, group, lam=0.01, lazy_batch=128, keep_stages=False):
    """Quantize several modules that share one damped H (n_store x n_store).

    modules: list of dicts with keys name, W (rows x n_store, device, stored basis), bits (int),
    and optionally B (rows x r), A (r x n_store), alpha.  One batched GPTQ sweep and one joint
    scale solve run over the concatenated rows with a per-row bit width; then each module is
    wrung against its own adapter and packed.  Returns {name: dict(codes, scales, packed, ...)}
    with codes/scales as views into the batched buffers.
    """
    n = H.shape[0]
    sizes = [m["W"].shape[0] for m in modules]
    W = torch.cat([m["W"] for m in modules]) if len(modules) > 1 else modules[0]["W"]
    bits_t = torch.cat([torch.full((r,), int(m["bits"]), dtype=torch.uint8, device=ctx.device)
                        for m, r in zip(modules, sizes)])
    rows = W.shape[0]
    codes = torch.empty(rows, n, dtype=torch.uint8, device=ctx.device)
    scales = torch.empty(rows, n // group, dtype=torch.float16, device=ctx.device)
    info = torch.zeros(2 + len(modules), dtype=torch.int32, device=ctx.device)
    wr.wr_gptq_sweep(ctx, W, H, bits_t, group, lazy_batch, codes, scales, info[0:1])
    stages = {}
    if keep_stages:
        stages["gptq_codes"], stages["gptq_scales"] = codes.clone(), scales.clone()
    wr.wr_wring_solve(ctx, H, bits_t, group, lam, codes, scales, info[1:2], target=W)
    if keep_stages:
        stages["joint_scales"] = scales.clone()
    out = {}
    r0 = 0
    for k, (m, r) in enumerate(zip(modules, sizes)):
        c, s, b = codes[r0:r0 + r], scales[r0:r0 + r], bits_t[r0:r0 + r]
        if m.get("B") is not None:
            wr.wr_wring_solve(ctx, H, b, group, lam, c, s, info[2 + k:3 + k], B=m["B"], A=m["A"],
                              alpha=m.get("alpha", m["A"].shape[0]), recode=True)
        res = {"codes": c, "scales": s, "packed": pack(ctx, c, s, int(m["bits"]), group), "rows": (r0, r0 + r),
               "bits": int(m["bits"])}
        for key, val in stages.items():
            res[key] = val[r0:r0 + r]
        out[m["name"]] = res
        r0 += r
    out["_dev_info"] = info
    return out


def container_bytes(entries, meta):
    """A safetensors-format container: an 8-byte little-endian header length, a JSON header naming
    each packed buffer (dtype U8, 1-D) and carrying `wringer_meta` (JSON text) under __metadata__,
    then the raw bytes in order.  entries: list of (name, host uint8 numpy array)."""
    import json
    import struct
    header = {"__metadata__": {"wringer_meta": json.dumps(meta, sort_keys=True)}}
    off = 0
    for name, buf in entries:
        header[name] = {"dtype": "U8", "shape": [int(buf.size)], "data_offsets": [off, off + int(buf.size)]}
        off += int(buf.size)
    text = json.dumps(header, separators=(",", ":")).encode()
    text += b" " * ((8 - len(text) % 8) % 8)
    return b"".join([struct.pack("<Q", len(text)), text] + [buf.tobytes() for _, buf in entries])
