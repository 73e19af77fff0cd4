"""Throughput of the per-linear-layer quantization solve on one MI355X.

Default workload: the whole 36-layer Qwen3-4B-shaped body (36 x 7 modules,
3 633 315 840 weights).  One step = for every layer and each of its three input
dimensions (2560: q k v gate up; 4096: o; 9728: down): H accumulation over
262144 calibration rows + finalize with the random-sign Hadamard rotation
(blocks of 512) and damping + rotation of the weights + factorisation and GPTQ
sweep of the stacked rows sharing that H + joint scales + the wring of every
module against its rank-128 adapter (nearest-point codes, joint scales) +
packing and unpacking of every module.  Inputs (weights, adapters, calibration
rows) are synthetic and resident in HBM before the timed region: the body's
calibration rows (309 GB) exceed the 288 GB of HBM, so `--calib-sets` distinct
per-layer calibration sets are kept resident and layer l reads set l mod
calib_sets (the work per layer does not depend on the values).  The metric is
weights quantized per second.  The timed steps run each input dimension's
solves on a stream of its own, the widest dimension's layers rotating over
three streams and buffer sets and the narrowest's alternating over two (six
streams), and every H accumulation waits for the previous one, so that two
never run at once.

Also reported: the roofline of the dominant kernel (the bf16 SYRK that
accumulates H: N n (n + 1) useful flops per call, timed live with HIP events on
the stream it runs on), a per-call breakdown of one separate untimed pass, and
the CPU oracle timed on a bounded sample of the same workload on the host cores.
`--workload q_proj` times one q_proj module (4096 x 2560) instead, with the
materializer, finisher variants, trellis quantizer and packed-module product
timed beside it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload body|q_proj] [--no-cpu-baseline]
       python bench.py --kernel-summary RESULTS_DB   (per-kernel table of a rocprofv3 kernel trace)
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

WORKLOAD = {
    "workload": "q_proj 4096x2560 bf16 (Student-t nu=5, std 0.02), X 131072x2560 bf16 (spectral + 1% outlier "
                "channels), 2-bit signed odd grid, group 64, fp16 scales, lazy batch 128, damping 0.01, "
                "rank-128 wring alpha 128, lambda 0.01, pack",
    "rows": 4096, "n": 2560, "calib_rows": 131072, "bits": 2, "group": 64, "lazy_batch": 128, "rank": 128,
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--workload", choices=("body", "q_proj"), default="body")
    p.add_argument("--layers", type=int, default=36, help="body: layers per step (the workload has 36)")
    p.add_argument("--calib-sets", type=int, default=4,
                   help="body: distinct per-layer calibration sets kept resident (layer l reads set l mod K)")
    p.add_argument("--no-breakdown", action="store_true", help="body: skip the untimed per-call breakdown pass")
    p.add_argument("--streams", type=int, choices=(1, 3, 4, 5, 6, 7, 8), default=7,
                   help="body: 3 runs each input dim's solves on a stream of its own (they overlap); 4 also "
                        "alternates the widest dim's layers between two streams and buffer sets, 5 between "
                        "three, 6 every dim's between two, 7 (the default) the widest dim's over three and the "
                        "narrowest dim's over two (six streams), 8 the widest dim's over four and the "
                        "narrowest dim's over two (seven); 1 runs every call in order")
    p.add_argument("--lag", type=int, default=0,
                   help="body, several streams: a stream starts layer l once the others have finished layer l - lag "
                        "(0: no coupling)")
    p.add_argument("--hw-queues", type=int, choices=range(1, 33), default=8, metavar="Q",
                   help="hardware queues HIP gives the process (GPU_MAX_HW_QUEUES, read when its runtime starts; "
                        "default 8): the body step's six streams and the default stream need seven, and two "
                        "streams that share a queue run one after the other")
    p.add_argument("--h-chain", choices=("none", "dim", "all"), default="all",
                   help="body, several streams: an H accumulation waits for the previous one of its input dim "
                        "(dim) or of any dim (all, the default: accumulations never run at once), or for "
                        "nothing but its own stream's work (none)")
    p.add_argument("--no-measures", action="store_true", help="body: skip the model cards' measures of layer 0")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=None, help="weight rows in the oracle sample")
    p.add_argument("--cpu-calib", type=int, default=None, help="calibration rows in the oracle sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="before the warmup, copy MIB mebibytes device to device once (a plain copy kernel of known "
                        "size, the yardstick for the FETCH_SIZE / WRITE_SIZE counters)")
    p.add_argument("--no-extras", action="store_true",
                   help="q_proj: time the solve step only (no materializer or finisher-variant timing)")
    p.add_argument("--extras-only", action="store_true",
                   help="q_proj: one untimed step (for H), then only the materializer and the finisher-variant timings")
    p.add_argument("--syrk", type=int, default=0, metavar="N",
                   help="time only the H accumulation over 262144 Gaussian calibration rows of input dim N (for "
                        "kernel counters; prints one JSON line and exits)")
    p.add_argument("--kernel-summary", metavar="RESULTS_DB", default=None,
                   help="print the per-kernel table of a rocprofv3 kernel trace (rocpd database) and exit")
    p.add_argument("--trace-steps", type=int, default=1,
                   help="with --kernel-summary: body steps the trace covers (warmup + timed + breakdown)")
    return p.parse_args()


def traffic_from_profile(name, key="bytes_per_launch"):
    """HBM bytes of the SYRK launches from a committed rocprofv3 counter summary, if it matches this source.

    The summary (profiles/<name>) holds `bytes_per_launch:` (FETCH_SIZE and WRITE_SIZE per dispatch, each
    scaled by what the counter reads for a plain copy of known size; for the body, summed over one step's
    launches) and `source_sha256:` of the kernel source it was taken on (k_hessian.hip followed by
    common.hpp, which holds its tile order); once the source has changed the figure no longer describes
    the kernel and None is returned.
    """
    path = os.path.join(ROOT, "profiles", name)
    csrc = os.path.join(ROOT, "post_bit_weight_amd", "csrc")
    try:
        rec = {}
        for line in open(path):
            if ":" in line and not line.startswith((" ", "#")):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
        digest = hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read()
                                         for f in ("k_hessian.hip", "common.hpp"))).hexdigest()
        if rec.get("source_sha256") != digest:
            return None
        return float(rec[key])
    except (OSError, ValueError, KeyError):
        return None


def cpu_baseline(X_host, W_host, B_host, A_host, cfg, n_rows=128, n_calib=8192):
    """The oracle, unchanged, on a bounded sample; extrapolated to the full workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    n, g, bits, rank = cfg["n"], cfg["group"], cfg["bits"], cfg["rank"]
    t0 = time.perf_counter()
    H0 = oracle.second_moment(X_host[:n_calib].astype(np.float64))
    t_h = time.perf_counter() - t0
    H, _ = oracle.damp(H0, 0.01)
    W = W_host[:n_rows].astype(np.float64)
    t0 = time.perf_counter()
    g0 = oracle.gptq_sweep(W, H, bits, g)
    t_sweep = time.perf_counter() - t0
    t0 = time.perf_counter()
    s1, _ = oracle.joint_scales(g0["codes"], bits, g, H, W, g0["scales"], 0.01)
    w = oracle.wring(g0["codes"], s1, bits, g, B_host[:n_rows].astype(np.float64), A_host.astype(np.float64),
                     float(rank), H, 0.01)
    oracle.pack(w["codes"], w["scales"], bits, g)
    t_rest = time.perf_counter() - t0
    # the factorisation inside gptq_sweep is done once per module; time it alone to split it off
    t0 = time.perf_counter()
    oracle.upper_cholesky_of_inverse(H)
    t_fact = time.perf_counter() - t0
    per_row = (t_sweep - t_fact + t_rest) / n_rows
    full = t_h * cfg["calib_rows"] / n_calib + t_fact + per_row * cfg["rows"]
    return {
        "value": cfg["rows"] * n / full, "unit": "weights/s", "cores": int(threads), "kind": "oracle",
        "sample": f"H over {n_calib} of {cfg['calib_rows']} calibration rows, sweep/joint/wring/pack over "
                  f"{n_rows} of {cfg['rows']} weight rows, one factorisation; extrapolated linearly "
                  f"(measured {t_h + t_sweep + t_rest + t_fact:.1f} s)",
    }


def time_materialize(wr, ctx, torch, reps=20):
    """The materializer (packed module -> bf16 weights, inverse rotation) on one layer's 2560-wide
    group of the 36-layer body: q, k, v, gate and up stacked, 25600 x 2560, 2-bit, group 64,
    Hadamard blocks of 512.  HBM-bound: algorithmic bytes = packed codes and scales read + bf16
    written, against the 8 TB/s peak."""
    rows, n, bits, g, m = 25600, 2560, 2, 64, 512
    code_bytes = rows * n * bits // 8
    gen = torch.Generator(device="cuda").manual_seed(20261208)
    buf = torch.randint(0, 256, (wr.packed_nbytes(rows, n, bits, g),), dtype=torch.uint8, device="cuda",
                        generator=gen)
    sc = (torch.rand(rows * (n // g), device="cuda", generator=gen) * 0.029 + 1e-3).to(torch.float16)
    buf[code_bytes:] = sc.view(torch.uint8)
    signs = (torch.randint(0, 2, (n,), device="cuda", generator=gen) * 2 - 1).to(torch.int8)
    out = torch.empty(rows, n, dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        wr.wr_materialize(ctx, buf, rows, n, bits, g, out, had_block=m, signs=signs)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(ctx.stream)
    for _ in range(reps):
        wr.wr_materialize(ctx, buf, rows, n, bits, g, out, had_block=m, signs=signs)
    e1.record(ctx.stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = buf.numel() + 2 * rows * n
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"{rows}x{n} 2-bit group {g}, inverse Hadamard blocks of {m}", "ms": ms,
            "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "bytes_per_launch": nbytes}


def time_finisher_gptq(wr, ctx, torch, H, W, B, A, bits_t, cfg, reps=5):
    """The finisher variants on the step's workload, from the first solve's codes and scales: GPTQ
    codes (wr_wring_solve with WR_RECODE_GPTQ: watered target, GPTQ sweep of it, joint scales) and
    searched block scales (WR_RECODE_SEARCH: watered target, 32 candidate scales per block).
    Each call is timed alone with HIP events on the library's stream."""
    rows, n, g, rank = cfg["rows"], cfg["n"], cfg["group"], cfg["rank"]
    c1 = torch.empty(rows, n, dtype=torch.uint8, device="cuda")
    s1 = torch.empty(rows, n // g, dtype=torch.float16, device="cuda")
    info = torch.zeros(3, dtype=torch.int32, device="cuda")
    wr.wr_gptq_sweep(ctx, W, H, bits_t, g, 128, c1, s1, info[0:1])
    wr.wr_wring_solve(ctx, H, bits_t, g, 0.01, c1, s1, info[1:2], target=W)
    codes, scales = torch.empty_like(c1), torch.empty_like(s1)
    out = {}
    for kind in ("gptq", "search"):
        times = []
        for k in range(reps + 2):
            codes.copy_(c1)
            scales.copy_(s1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(ctx.stream)
            wr.wr_wring_solve(ctx, H, bits_t, g, 0.01, codes, scales, info[2:3], B=B, A=A, alpha=float(rank),
                              recode=kind)
            e1.record(ctx.stream)
            torch.cuda.synchronize()
            if k >= 2:
                times.append(e0.elapsed_time(e1))
        if int(info.abs().sum().item()) != 0:
            raise RuntimeError(f"dev_info reports a failure in the {kind} finisher: {info.tolist()}")
        ms = sum(times) / len(times)
        out[kind] = {"ms": ms, "weights_per_s": rows * n / (ms * 1e-3)}
    return {"workload": f"wring with GPTQ codes / with searched block scales, {rows}x{n}, rank {rank}",
            "ms": out["gptq"]["ms"], "weights_per_s": out["gptq"]["weights_per_s"], "scale_search": out["search"]}


PEAK_VALU_OPS = 256 * 64 * 2.4e9  # fp32 lane operations per second without packing: 256 CUs x 64 lanes x 2.4 GHz


def time_trellis(wr, ctx, torch, reps=5):
    """Trellis-coded quantization (Viterbi search) of one layer's 2560-wide group, 25600 x 2560
    targets in level units (Student-t, std 1.5), 8-state trellis, cosets of 2 (2 bits/weight).
    Bound by VALU issue: per weight and state the forward pass evaluates 2 branches x 2 coset
    values (subtract, multiply, min: 3 ops each) and keeps the cheaper of 2 candidates (2 adds,
    compare, select), 16 ops, i.e. 128 per weight; the traceback adds about 12 per weight."""
    from post_bit_weight_amd import synth
    rows, n, log2s = 25600, 2560, 3
    T = synth.student_t((rows, n), seed=20261230, std=1.5, device="cuda")
    vals = synth.trellis8_values(device="cuda")
    codes = torch.empty(rows, n, dtype=torch.uint8, device="cuda")
    cost = torch.empty(rows, dtype=torch.float64, device="cuda")
    for _ in range(2):
        wr.wr_trellis_quantize(ctx, T, log2s, vals, codes, None, cost)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(ctx.stream)
    for _ in range(reps):
        wr.wr_trellis_quantize(ctx, T, log2s, vals, codes, None, cost)
    e1.record(ctx.stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    ops = 140.0 * rows * n
    achieved = ops / (ms * 1e-3)
    return {"workload": f"trellis {rows}x{n}, 8 states, cosets of 2 (2 bits/weight)", "ms": ms,
            "weights_per_s": rows * n / (ms * 1e-3), "bound": "alu", "achieved": achieved / 1e12,
            "peak": PEAK_VALU_OPS / 1e12, "unit": "Tops/s", "frac": achieved / PEAK_VALU_OPS,
            "algorithmic_ops_per_weight": 140}


def queued_ms(torch, ctx, fn, reps):
    """GPU time per call of fn with the calls queued back to back: a spin kernel holds the stream
    while the host enqueues the calls (so host-side overhead, larger than a few-microsecond call,
    does not show as idle GPU time); checks that the spin outlasted the enqueueing."""
    cycles = 20_000_000
    for _ in range(6):
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record(ctx.stream)
        torch.cuda._sleep(cycles)
        s1.record(ctx.stream)
        e0.record(ctx.stream)
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        host_ms = (time.perf_counter() - t0) * 1e3
        e1.record(ctx.stream)
        torch.cuda.synchronize()
        if s0.elapsed_time(s1) > 1.2 * host_ms:
            return e0.elapsed_time(e1) / reps
        cycles *= 2
    raise RuntimeError("the spin kernel did not cover the host's enqueueing")


def time_gemv(wr, ctx, torch, reps=50):
    """The packed-module product (decode-time use of the container) on one layer's 2560-wide group,
    25600 x 2560, 2-bit, group 64, blocks of 512, one input vector.  HBM-bound: algorithmic bytes
    = the packed codes and scales read once (the vector and the outputs are 0.6 % more).  Timed
    with HIP events over `reps` calls queued back to back (each call: the input rotation and the
    product)."""
    rows, n, bits, g, m = 25600, 2560, 2, 64, 512
    gen = torch.Generator(device="cuda").manual_seed(20261240)
    code_bytes = rows * n * bits // 8
    buf = torch.randint(0, 256, (wr.packed_nbytes(rows, n, bits, g),), dtype=torch.uint8, device="cuda", generator=gen)
    sc = (torch.rand(rows * (n // g), device="cuda", generator=gen) * 0.029 + 1e-3).to(torch.float16)
    buf[code_bytes:] = sc.view(torch.uint8)
    signs = (torch.randint(0, 2, (n,), device="cuda", generator=gen) * 2 - 1).to(torch.int8)
    x = torch.randn(1, n, device="cuda", generator=gen)
    y = torch.empty(1, rows, dtype=torch.float32, device="cuda")
    def call():
        wr.wr_packed_gemv(ctx, buf, rows, n, bits, g, x, y, had_block=m, signs=signs)
    for _ in range(3):
        call()
    ms = queued_ms(torch, ctx, call, reps)
    nbytes = buf.numel()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"packed product {rows}x{n} 2-bit group {g}, blocks of {m}, 1 vector", "ms_per_call": ms,
            "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "bytes_per_call": nbytes}


def progress(msg):
    print(f"bench.py: {msg}", file=sys.stderr, flush=True)


def main_q_proj(args):
    import numpy as np
    import torch
    from post_bit_weight_amd import _lib as wr
    from post_bit_weight_amd import synth

    cfg = WORKLOAD
    rows, n, N, g, bits, rank = cfg["rows"], cfg["n"], cfg["calib_rows"], cfg["group"], cfg["bits"], cfg["rank"]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ctx = wr.Context(0)
    st = ctx.stream

    progress("drawing the synthetic inputs")
    src = synth.SpectralSource(n, seed=20261204, device="cuda", outlier_frac=0.01)
    X = torch.cat([src.chunk(k, 16384) for k in range(N // 16384)])
    W = synth.student_t((rows, n), seed=20261205, device="cuda", dtype=torch.bfloat16)
    B = synth.gaussian((rows, rank), 0.01, seed=20261206, device="cuda", dtype=torch.bfloat16)
    A = synth.gaussian((rank, n), 0.01, seed=20261207, device="cuda", dtype=torch.bfloat16)

    S = torch.empty(n, n, dtype=torch.float64, device=dev)
    H = torch.empty(n, n, dtype=torch.float32, device=dev)
    delta = torch.empty(1, dtype=torch.float32, device=dev)
    bits_t = torch.full((rows,), bits, dtype=torch.uint8, device=dev)
    codes = torch.empty(rows, n, dtype=torch.uint8, device=dev)
    scales = torch.empty(rows, n // g, dtype=torch.float16, device=dev)
    info = torch.zeros(3, dtype=torch.int32, device=dev)
    packed = torch.empty(wr.packed_nbytes(rows, n, bits, g), dtype=torch.uint8, device=dev)
    ws = max(wr.wr_workspace_bytes(wr.WR_OP_HESSIAN, N, n), wr.wr_workspace_bytes(wr.WR_OP_GPTQ, rows, n, g, 0, 128),
             wr.wr_workspace_bytes(wr.WR_OP_FINALIZE, 0, n),
             wr.wr_workspace_bytes(wr.WR_OP_WRING, rows, n, g, rank, 0))
    ctx.ensure_workspace(ws)

    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src_buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst_buf = torch.empty_like(src_buf)
        dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf

    stages = ["hessian", "finalize", "gptq", "joint", "wring", "pack"]

    def step(ev=None, all_stages=True):
        # a timing event between two kernels opens a gap of a few microseconds on the stream, so
        # the timed steps mark only the H accumulation (the roofline's kernel); the breakdown by
        # stage comes from separate steps
        def mark(i):
            if ev is not None and (all_stages or i < 2):
                ev[i].record(st)
        mark(0)
        wr.wr_hessian_accumulate(ctx, X, S, zero=True)
        mark(1)
        wr.wr_hessian_finalize(ctx, S, N, 0.01, H, delta)
        mark(2)
        wr.wr_gptq_sweep(ctx, W, H, bits_t, g, 128, codes, scales, info[0:1])
        mark(3)
        wr.wr_wring_solve(ctx, H, bits_t, g, 0.01, codes, scales, info[1:2], target=W)
        mark(4)
        wr.wr_wring_solve(ctx, H, bits_t, g, 0.01, codes, scales, info[2:3], B=B, A=A, alpha=float(rank), recode=True)
        mark(5)
        wr.wr_pack(ctx, codes, scales, bits, g, packed)
        mark(6)

    progress("warmup")
    for _ in range(1 if args.extras_only else args.warmup):
        step()
    torch.cuda.synchronize()
    if int(info.abs().sum().item()) != 0:
        raise RuntimeError(f"dev_info reports a failure: {info.tolist()}")
    if args.extras_only:
        progress("timing the materializer and the GPTQ-codes finisher")
        print(json.dumps({"materialize": time_materialize(wr, ctx, torch),
                          "finisher_gptq": time_finisher_gptq(wr, ctx, torch, H, W, B, A, bits_t, cfg),
                          "trellis": time_trellis(wr, ctx, torch), "gemv": time_gemv(wr, ctx, torch)}), flush=True)
        return

    progress(f"timing {args.steps} steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k], all_stages=False)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / args.steps
    h_ms = float(np.mean([evs[k][0].elapsed_time(evs[k][1]) for k in range(args.steps)]))
    progress("stage breakdown (separate, untimed steps)")
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(min(args.steps, 3))]
    for e in sev:
        step(e)
    torch.cuda.synchronize()
    per_stage = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in sev])) for i, name in enumerate(stages)}
    per_stage["hessian"] = h_ms

    flops_h = float(N) * n * (n + 1)
    t_h = per_stage["hessian"] * 1e-3
    achieved = flops_h / t_h / 1e12
    traffic = traffic_from_profile("syrk_bf16_q_proj_traffic.txt")
    line = {
        "metric": "weights quantized/s (H accum+GPTQ sweep+wring); % MFMA/HBM peak, 1 GPU",
        "value": rows * n / (ms * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-mfma/fp32",
        "data": "synthetic",
        "config": {**cfg, "parallelism": "none (1 GPU)"},
        "roofline": {
            "kernel": "syrk_bf16 (H accumulation incl. its split-K reduction)",
            "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
            "algorithmic_flops_per_launch": flops_h, "launch_ms": per_stage["hessian"],
        },
        "stage_ms": per_stage,
    }
    if not args.no_extras:
        progress("timing the materializer")
        line["materialize"] = time_materialize(wr, ctx, torch)
        progress("timing the GPTQ-codes finisher")
        line["finisher_gptq"] = time_finisher_gptq(wr, ctx, torch, H, W, B, A, bits_t, cfg)
        progress("timing the trellis quantizer")
        line["trellis"] = time_trellis(wr, ctx, torch)
        progress("timing the packed-module product")
        line["gemv"] = time_gemv(wr, ctx, torch)
    if not args.no_cpu_baseline:
        progress("timing the oracle on a bounded sample")
        Xh = X[: args.cpu_calib].float().cpu().numpy()
        Wh = W.float().cpu().numpy()
        Bh = B.float().cpu().numpy()
        Ah = A.float().cpu().numpy()
        line["cpu_baseline"] = cpu_baseline(Xh, Wh, Bh, Ah, cfg, args.cpu_rows or 128, args.cpu_calib or 8192)
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------- body
BODY = {"layers": 36, "calib_rows": 262144, "chunk": 16384, "had_block": 512, "group": 64, "rank": 128,
        "lazy_batch": 128, "damp": 0.01, "lam": 0.01, "seed": 2026}


def body_flops_syrk(layers, calib_rows, dims):
    return float(layers) * sum(float(calib_rows) * n * (n + 1) for n in dims)


class BodyInputs:
    """Everything one body step reads and writes, allocated and drawn before the timed region.

    Per layer and input dim: the stacked weights of the modules sharing that H (bf16, module rows
    consecutive, as the batched sweep takes them), each module's adapter B, A, the per-row bit
    widths; outputs codes/scales per layer (the result), the packed module and its unpacked codes
    and scales (the round trip).  Calibration rows: `calib_sets` resident sets per input dim."""

    def __init__(self, torch, wr, body, synth, layers, calib_sets, cfg, log):
        dev = torch.device("cuda", 0)
        self.layers, self.P, self.cfg = layers, calib_sets, cfg
        N, chunk, g, r, seed = cfg["calib_rows"], cfg["chunk"], cfg["group"], cfg["rank"], cfg["seed"]
        self.dims = body.DIMS
        self.X = {n: [] for n in self.dims}
        for n in self.dims:
            src = body.CalibrationStream(n, seed * 31 + n, dev)
            for p in range(calib_sets):
                X = torch.empty(N, n, dtype=torch.bfloat16, device=dev)
                for k in range(N // chunk):
                    X[k * chunk:(k + 1) * chunk] = src.chunk(p, k, chunk)
                self.X[n].append(X)
            log(f"calibration sets drawn for input dim {n}")
        self.signs = {n: synth.signs(n, seed=seed * 7 + n, device=dev) for n in self.dims}
        self.S = {n: torch.empty(n, n, dtype=torch.float64, device=dev) for n in self.dims}
        self.H = {n: torch.empty(n, n, dtype=torch.float32, device=dev) for n in self.dims}
        self.none = {n: torch.empty(0, n, dtype=torch.bfloat16, device=dev) for n in self.dims}
        self.delta = {n: torch.empty(1, dtype=torch.float32, device=dev) for n in self.dims}
        names = [m[0] for m in body.MODULES]
        self.groups = []
        for layer in range(layers):
            per = {}
            for n in self.dims:
                mods = [(name, rows) for name, rows, dim in body.MODULES if dim == n]
                total = sum(rows for _, rows in mods)
                W = torch.empty(total, n, dtype=torch.bfloat16, device=dev)
                bits = torch.empty(total, dtype=torch.uint8, device=dev)
                entries, r0 = [], 0
                for name, rows in mods:
                    ms = seed * 100003 + 1000 * layer + 10 * names.index(name)
                    W[r0:r0 + rows] = synth.student_t((rows, n), seed=ms, device=dev, dtype=torch.bfloat16)
                    b = body.module_bits(layer, name, cfg["layers"])
                    bits[r0:r0 + rows] = b
                    entries.append(dict(
                        name=name, r0=r0, r1=r0 + rows, bits=b,
                        B=synth.gaussian((rows, r), 0.01, seed=ms + 1, device=dev, dtype=torch.bfloat16),
                        A=synth.gaussian((r, n), 0.01, seed=ms + 2, device=dev, dtype=torch.bfloat16),
                        packed=torch.empty(wr.packed_nbytes(rows, n, b, g), dtype=torch.uint8, device=dev)))
                    r0 += rows
                per[n] = dict(W=W, bits=bits, mods=entries,
                              codes=torch.empty(total, n, dtype=torch.uint8, device=dev),
                              scales=torch.empty(total, n // g, dtype=torch.float16, device=dev),
                              ucodes=torch.empty(total, n, dtype=torch.uint8, device=dev),
                              uscales=torch.empty(total, n // g, dtype=torch.float16, device=dev),
                              info=torch.full((2 + len(entries),), -7, dtype=torch.int32, device=dev))
            self.groups.append(per)
        rows_max = {n: self.groups[0][n]["W"].shape[0] for n in self.dims}
        self.Wst = {n: torch.empty(rows_max[n], n, dtype=torch.float32, device=dev) for n in self.dims}
        # per input dim, the buffer sets its layers cycle through (S, H, rotated weights, delta): one,
        # or two for a dim whose layers alternate between two streams (add_set)
        self.sets = {n: [dict(S=self.S[n], H=self.H[n], Wst=self.Wst[n], delta=self.delta[n])] for n in self.dims}
        self._dev, self._rows_max = dev, rows_max
        self.weights = sum(int(v["W"].numel()) for per in self.groups for v in per.values())
        self.payload = sum(int(m["packed"].numel()) for per in self.groups for v in per.values() for m in v["mods"])
        ws = 0
        for n in self.dims:
            rows = rows_max[n]
            ws = max(ws, wr.wr_workspace_bytes(wr.WR_OP_HESSIAN, N, n),
                     wr.wr_workspace_bytes(wr.WR_OP_FINALIZE, 0, n),
                     wr.wr_workspace_bytes(wr.WR_OP_GPTQ, rows, n, g, 0, cfg["lazy_batch"]),
                     wr.wr_workspace_bytes(wr.WR_OP_WRING, rows, n, g, r, 0))
        self.ws_bytes = ws

    def add_set(self, torch, n):
        """A second buffer set for input dim n (layers then alternate between the two)."""
        dev = self._dev
        self.sets[n].append(dict(S=torch.empty(n, n, dtype=torch.float64, device=dev),
                                 H=torch.empty(n, n, dtype=torch.float32, device=dev),
                                 Wst=torch.empty(self._rows_max[n], n, dtype=torch.float32, device=dev),
                                 delta=torch.empty(1, dtype=torch.float32, device=dev)))


def body_step(wr, ctxs, I, mark=None, lag=0, h_chain=None):
    """One pass of the whole solve over the body.  ctxs: one library context for every call (they run
    in order on its stream), or a dict (input dim, buffer set) -> context: the solves of a dim's layers
    that use set k of its buffers run on that context's stream and overlap with the others (a set's
    buffers are only touched on its own stream, so the streams share nothing; with two sets a dim's
    even and odd layers alternate).  With lag > 0 a stream starts layer l only after every other
    stream has finished layer l - lag.  h_chain "dim" (or "all") makes every H
    accumulation wait for the previous one of its input dim (of any dim), so that accumulations on
    different streams never run at once.  mark(kind, n, stream) is called between library calls when
    given (it records timing events on the stream of the call)."""
    import torch
    single = not isinstance(ctxs, dict)
    cfg = I.cfg
    g, lam, hb, N = cfg["group"], cfg["lam"], cfg["had_block"], cfg["calib_rows"]
    m = mark or (lambda kind, n, stream: None)
    done = []  # per layer: {n: event at the end of layer on its stream}
    chain = h_chain if not single and h_chain != "none" else None
    h_last = {}  # chain key -> event at the end of the last H accumulation
    for layer in range(I.layers):
        p = layer % I.P
        if not single and lag > 0:
            done.append({})
        for n in I.dims:
            k = 0 if single else layer % len(I.sets[n])
            buf = I.sets[n][k]
            ctx = ctxs if single else ctxs[(n, k)]
            if not single and lag > 0 and layer >= lag:
                for n2, ev in done[layer - lag].items():
                    if n2 != n:
                        ctx.stream.wait_event(ev)
            G = I.groups[layer][n]
            rows = G["W"].shape[0]
            S, H, Wst = buf["S"], buf["H"], buf["Wst"][:rows]
            key = n if chain == "dim" else 0
            if chain and key in h_last:
                ctx.stream.wait_event(h_last[key])
            wr.wr_hessian_accumulate(ctx, I.none[n], S, zero=True)          # S = 0
            m("hessian", n, ctx.stream)
            wr.wr_hessian_accumulate(ctx, I.X[n][p], S)
            m("finalize", n, ctx.stream)
            if chain:
                ev = torch.cuda.Event()
                ev.record(ctx.stream)
                h_last[key] = ev
            wr.wr_hessian_finalize(ctx, S, N, cfg["damp"], H, buf["delta"], hb, I.signs[n])
            m("rotate", n, ctx.stream)
            with torch.cuda.stream(ctx.stream):
                Wst.copy_(G["W"])                                                # widen to fp32
            wr.wr_hadamard_rotate(ctx, Wst, hb, I.signs[n], wr.WR_ROT_ROWS)
            m("gptq", n, ctx.stream)
            wr.wr_gptq_sweep(ctx, Wst, H, G["bits"], g, cfg["lazy_batch"], G["codes"], G["scales"],
                             G["info"][0:1])
            m("joint", n, ctx.stream)
            wr.wr_wring_solve(ctx, H, G["bits"], g, lam, G["codes"], G["scales"], G["info"][1:2], target=Wst)
            for kk, mod in enumerate(G["mods"]):
                sl = slice(mod["r0"], mod["r1"])
                m("wring", n, ctx.stream)
                wr.wr_wring_solve(ctx, H, G["bits"][sl], g, lam, G["codes"][sl], G["scales"][sl],
                                  G["info"][2 + kk:3 + kk], B=mod["B"], A=mod["A"], alpha=float(cfg["rank"]),
                                  recode=True)
                m("pack", n, ctx.stream)
                wr.wr_pack(ctx, G["codes"][sl], G["scales"][sl], mod["bits"], g, mod["packed"])
                m("unpack", n, ctx.stream)
                wr.wr_unpack(ctx, mod["packed"], mod["r1"] - mod["r0"], n, mod["bits"], g, G["ucodes"][sl],
                             G["uscales"][sl])
            m("end", n, ctx.stream)
            if not single and lag > 0:
                ev = torch.cuda.Event()
                ev.record(ctx.stream)
                done[layer][n] = ev


def body_check(torch, I):
    """After a step: every dev_info is 0 and every module's unpacked codes and scales equal the codes
    and scales it was packed from."""
    for layer, per in enumerate(I.groups):
        for n, G in per.items():
            info = G["info"].cpu().tolist()
            if any(v != 0 for v in info):
                raise RuntimeError(f"layer {layer}, input dim {n}: dev_info {info}")
            if not (torch.equal(G["ucodes"], G["codes"]) and
                    torch.equal(G["uscales"].view(torch.int16), G["scales"].view(torch.int16))):
                raise RuntimeError(f"layer {layer}, input dim {n}: pack/unpack round trip differs")


def body_measures(wr, ctx, I, torch, layer=0):
    """The model cards' measures for every module of one layer (off the timed path): grid distance of
    the parent and the filled weights, GPTQ-vs-nearest code disagreement without and with the adapter,
    one-ulp moves of the fp16 projection.  Returns {module: {measure: value}} and the weight-averaged
    values."""
    from post_bit_weight_amd import measures, pipeline
    cfg = I.cfg
    g, lam, hb, N = cfg["group"], cfg["lam"], cfg["had_block"], cfg["calib_rows"]
    per, tot, wsum = {}, {}, 0
    for n in I.dims:
        G = I.groups[layer][n]
        wr.wr_hessian_accumulate(ctx, I.X[n][layer % I.P], I.S[n], zero=True)
        H, _ = pipeline.finalize_hessian(ctx, I.S[n], N, cfg["damp"], n, hb, I.signs[n])
        mods = [dict(name=m["name"], bits=m["bits"], W=pipeline.prepare_weights(ctx, G["W"][m["r0"]:m["r1"]], n, hb,
                                                                                I.signs[n]))
                for m in G["mods"]]
        res = pipeline.solve_group(ctx, mods, H, g, lam, cfg["lazy_batch"], keep_stages=True)
        for m, mod in zip(G["mods"], mods):
            r = res[m["name"]]
            bits_t = G["bits"][m["r0"]:m["r1"]]
            vals = measures.module_measures(ctx, H, mod["W"], bits_t, g, lam, r["gptq_codes"], r["joint_scales"],
                                            m["B"], m["A"], float(cfg["rank"]))
            per[m["name"]] = vals
            w = mod["W"].numel()
            wsum += w
            for k, v in vals.items():
                tot[k] = tot.get(k, 0.0) + v * w
        del res, mods, H
    return per, {k: v / wsum for k, v in tot.items()}


def cpu_baseline_body(I, body, torch, n_rows=2, h_rows=None):
    """The oracle, unchanged, on a bounded sample of the body; extrapolated to the 36 layers.

    Per input dim (layer 0): H over h_rows calibration rows of the resident set, the fp64 rotation of
    H, damping, the GPTQ sweep (with its factorisation), joint scales, wring and packing of n_rows rows
    of the group's first module, and (2560, 4096) the factorisation alone.  Per layer: H scaled to
    262144 rows + rotation + factorisation + per-row costs x the group's rows.  At 9728 the per-row
    sweep cost is the 4096 one scaled by n^2 (the factorisation at 9728 is timed once, inside the
    sweep call)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    cfg = I.cfg
    g, hb, lam, r = cfg["group"], cfg["had_block"], cfg["lam"], cfg["rank"]
    per_layer, measured, sweep_row = 0.0, 0.0, {}
    parts = []
    for n in I.dims:
        hr = h_rows or (512 if n > 4096 else 1024)
        G = I.groups[0][n]
        mod = G["mods"][0]
        Xh = I.X[n][0][:hr].float().cpu().numpy().astype(np.float64)
        sd = I.signs[n].double().cpu().numpy()
        W = G["W"][:n_rows].float().cpu().numpy().astype(np.float64)
        B = mod["B"][:n_rows].float().cpu().numpy().astype(np.float64)
        A = mod["A"].float().cpu().numpy().astype(np.float64)
        bits = mod["bits"]
        t0 = time.perf_counter()
        H0 = oracle.second_moment(Xh)
        t_h = time.perf_counter() - t0
        t0 = time.perf_counter()
        H0 = oracle.rotate_sym(H0, hb, sd)
        t_rot = time.perf_counter() - t0
        H, _ = oracle.damp(H0, cfg["damp"])
        Wr = oracle.rotate_rows(W, hb, sd)
        t0 = time.perf_counter()
        gq = oracle.gptq_sweep(Wr, H, bits, g)
        t_sweep = time.perf_counter() - t0
        t0 = time.perf_counter()
        s1, _ = oracle.joint_scales(gq["codes"], bits, g, H, Wr, gq["scales"], lam)
        w = oracle.wring(gq["codes"], s1, bits, g, B, A, float(r), H, lam)
        oracle.pack(w["codes"], w["scales"], bits, g)
        t_rest = time.perf_counter() - t0
        t_fact = None
        if n <= 4096:
            t0 = time.perf_counter()
            oracle.upper_cholesky_of_inverse(H)
            t_fact = time.perf_counter() - t0
            sweep_row[n] = max(t_sweep - t_fact, 0.0) / n_rows
        else:
            sweep_row[n] = sweep_row[4096] * (n / 4096.0) ** 2
            t_fact = max(t_sweep - n_rows * sweep_row[n], 0.0)
        rows = G["W"].shape[0]
        per_layer += t_h * cfg["calib_rows"] / hr + t_rot + t_fact + rows * (sweep_row[n] + t_rest / n_rows)
        measured += t_h + t_rot + t_sweep + t_rest + (t_fact if n <= 4096 else 0.0)
        parts.append(f"dim {n}: H over {hr} rows, {n_rows} weight rows")
    total = per_layer * cfg["layers"]
    weights = sum(rows * n for _, rows, n in body.MODULES) * cfg["layers"]
    return {"value": weights / total, "unit": "weights/s", "cores": int(threads), "kind": "oracle",
            "sample": "layer 0 of the body, per input dim: H over a few calibration rows, the fp64 rotation of H, "
                      "damping, factorisation, GPTQ sweep, joint scales, wring and packing of a few weight rows ("
                      + "; ".join(parts) + "); extrapolated linearly to 262144 calibration rows, every row of the "
                      f"layer and 36 layers (measured {measured:.1f} s)"}


def main_body(args):
    import numpy as np
    import torch
    from post_bit_weight_amd import _lib as wr
    from post_bit_weight_amd import body, synth

    cfg = dict(BODY)
    layers = args.layers
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ctx = wr.Context(0)
    st = ctx.stream

    progress(f"drawing the synthetic inputs ({args.calib_sets} resident calibration sets, {layers} layers)")
    I = BodyInputs(torch, wr, body, synth, layers, args.calib_sets, cfg, progress)
    ctx.ensure_workspace(I.ws_bytes)
    # the timed steps' contexts: one, or one per input dim and buffer set on streams of their own
    # (default priority); with 4 (5, 7) streams the widest dim's layers rotate over two (three), with 7
    # the narrowest dim's alternate over two
    ctxs = ctx
    if args.streams > 1:
        if args.streams in (4, 5, 7, 8):
            I.add_set(torch, max(I.dims))
        if args.streams in (5, 7, 8):
            I.add_set(torch, max(I.dims))
        if args.streams == 8:
            I.add_set(torch, max(I.dims))
        if args.streams in (7, 8):
            I.add_set(torch, min(I.dims))
        if args.streams == 6:
            for n in I.dims:
                I.add_set(torch, n)
        ctxs = {(n, k): wr.Context(0, stream=torch.cuda.Stream(dev)) for n in I.dims for k in range(len(I.sets[n]))}
        for c in ctxs.values():
            c.ensure_workspace(I.ws_bytes)
    torch.cuda.synchronize()

    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src_buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst_buf = torch.empty_like(src_buf)
        dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf

    progress(f"warmup ({args.warmup} steps)")
    for _ in range(args.warmup):
        body_step(wr, ctxs, I, lag=args.lag, h_chain=args.h_chain)
    torch.cuda.synchronize()
    if args.warmup:
        body_check(torch, I)

    # timed steps: events only around the H accumulation (the roofline's kernel), recorded on the
    # stream the accumulation runs on
    progress(f"timing {args.steps} steps")
    syrk = []

    def mark_syrk(kind, n, stream):
        if kind in ("hessian", "finalize"):
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            syrk.append((kind, n, e))

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        body_step(wr, ctxs, I, mark_syrk, lag=args.lag, h_chain=args.h_chain)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    progress("checking dev_info and the pack/unpack round trips")
    body_check(torch, I)
    ms = elapsed * 1e3 / args.steps
    h_ms = {n: 0.0 for n in I.dims}
    for (k0, n0, e0), (k1, n1, e1) in zip(syrk[0::2], syrk[1::2]):
        assert k0 == "hessian" and k1 == "finalize" and n0 == n1
        h_ms[n0] += e0.elapsed_time(e1) / args.steps
    N = cfg["calib_rows"]
    flops = {n: float(layers) * N * n * (n + 1) for n in I.dims}
    syrk_ms = sum(h_ms.values())
    achieved = sum(flops.values()) / (syrk_ms * 1e-3) / 1e12

    stage = None
    same_as_one_stream = None
    if not args.no_breakdown:
        progress("per-call breakdown (one separate, untimed step, every call in order on one stream)")
        evs = []

        def mark_all(kind, n, stream):
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            evs.append((kind, n, e))

        timed = [(G["codes"].clone(), G["scales"].clone()) for per in I.groups for G in per.values()]
        body_step(wr, ctx, I, mark_all)
        torch.cuda.synchronize()
        # the timed steps' codes and scales must equal the in-order step's bit for bit (the kernels are
        # deterministic; a difference would mean the streams raced)
        redo = [(layer, n, G["codes"], G["scales"]) for layer, per in enumerate(I.groups) for n, G in per.items()]
        diff = []
        for (c0, s0), (layer, n, c1, s1) in zip(timed, redo):
            dc = int((c0 != c1).sum())
            ds = int((s0.view(torch.int16) != s1.view(torch.int16)).sum())
            if dc or ds:
                diff.append(f"layer {layer} dim {n}: {dc} codes, {ds} scales")
        same_as_one_stream = not diff
        del timed
        if diff:
            raise RuntimeError("the timed steps' codes or scales differ from the in-order step's: " + "; ".join(diff[:12]))
        stage = {}
        for (k0, n0, e0), (_, _, e1) in zip(evs[:-1], evs[1:]):
            if k0 == "end":
                continue
            stage[k0] = stage.get(k0, 0.0) + e0.elapsed_time(e1)

    traffic = traffic_from_profile("syrk_bf16_body_traffic.txt", "bytes_per_step") if layers == 36 else None
    w_desc = (f"36-layer Qwen3-4B-shaped body ({layers} layers timed): q 4096x2560, k/v 1024x2560, gate/up "
              "9728x2560, o 2560x4096, down 2560x9728 bf16 (Student-t nu=5, std 0.02); per layer one H per input "
              "dim from 262144 calibration rows (spectral + 1% outlier channels; post-SwiGLU-like product model "
              "for 9728), random-sign Hadamard rotation blocks of 512, damping 0.01; batched GPTQ sweep per H "
              "(lazy batch 128), joint scales lambda 0.01, rank-128 wring alpha 128 per module, 2/3-bit mix "
              "(3-bit v, o, down, and k in layers 0-17), group 64, fp16 scales; pack + unpack round trip of every "
              "module")
    line = {
        "metric": "weights quantized/s (H accum+GPTQ sweep+wring); % MFMA/HBM peak, 1 GPU",
        "value": I.weights / (ms * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-mfma/fp32/fp64",
        "data": "synthetic",
        "config": {"workload": w_desc, "layers": layers, "weights": I.weights, "calib_rows_per_H": N,
                   "calib_sets_resident": args.calib_sets, "had_block": cfg["had_block"], "group": cfg["group"],
                   "rank": cfg["rank"], "lambda": cfg["lam"], "payload_bytes": I.payload,
                   "bits_per_weight": 8.0 * I.payload / I.weights, "parallelism": "none (1 GPU)",
                   "streams": args.streams, "layer_lag": args.lag,
                   "h_chain": args.h_chain, "hw_queues": os.environ.get("GPU_MAX_HW_QUEUES")},
        "roofline": {
            "kernel": "syrk_bf16 (H accumulation incl. its split-K reduction), all launches of a step",
            "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
            "algorithmic_flops_per_step": sum(flops.values()), "syrk_ms_per_step": syrk_ms,
            "per_input_dim": {str(n): {"ms": h_ms[n], "tflops": flops[n] / (h_ms[n] * 1e-3) / 1e12,
                                       "frac": flops[n] / (h_ms[n] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
                              for n in I.dims},
        },
    }
    if stage is not None:
        line["stage_ms"] = stage
        line["timed_equals_in_order"] = same_as_one_stream
        # the same launches timed alone: the breakdown pass runs every call in order on one stream
        excl = sum(flops.values()) / (stage["hessian"] * 1e-3) / 1e12
        line["roofline"]["exclusive"] = {
            "note": "breakdown pass, one stream (no other work on the GPU during the H accumulation)",
            "syrk_ms_per_step": stage["hessian"], "achieved": excl, "frac": excl / PEAK_BF16_TFLOPS}
        # HBM-bound steps against the stage times of the breakdown pass (a stage holds every kernel of
        # its calls, so the sweep's and the recode's figures are lower bounds; the per-kernel figures
        # are in the kernel-trace summary)
        work = body_work(layers)

        def hbm(key, st, note):
            gbs = work[key] / (stage[st] * 1e-3) / 1e9
            return {"bytes_per_step": work[key], "stage_ms": stage[st], "achieved": gbs, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "note": note}
        line["stage_rooflines"] = {
            "sweep": hbm("sweep", "gptq", "W fp32 read, codes and scales written, M's upper half read, per H; "
                         "the stage also holds the fp64 factorisation"),
            "recode": hbm("recode", "wring", "codes in and out and the scales of the nearest-point recode; the "
                          "stage also holds the Gram/RHS products and the per-row solves"),
            "pack": hbm("pack", "pack", "codes and scales read, packed stream and scales written"),
            "finalize": hbm("finalize", "finalize", "the two fp64 rotation passes of H: S read (mirrored), T written "
                            "and read, H fp32 written; the stage also holds the trace"),
            "rotate": hbm("rotate", "rotate", "the weights' rotation: fp32 read and written"),
            "unpack": hbm("unpack", "unpack", "packed stream and scales read, codes and scales written"),
        }
    if not args.no_measures:
        progress("the model cards' measures for layer 0 (untimed)")
        per, mean = body_measures(wr, ctx, I, torch)
        line["measures_layer0"] = {"weighted_mean": mean, "per_module": per}
    if not args.no_cpu_baseline:
        progress("timing the oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline_body(I, body, torch, n_rows=args.cpu_rows or 2, h_rows=args.cpu_calib)
    print(json.dumps(line), flush=True)


def body_work(layers):
    """Algorithmic work of one body step over `layers` layers, per step of the path: bf16 MFMA flops
    (syrk, gram), fp64 flops (chol, rowsolve) and HBM bytes (sweep, recode, pack)."""
    from post_bit_weight_amd import body as _body
    N, g = BODY["calib_rows"], BODY["group"]
    groups = {}
    for name, rows, n in _body.MODULES:
        groups.setdefault(n, []).append((name, rows))
    work = {"syrk": 0.0, "chol": 0.0, "sweep": 0.0, "recode": 0.0, "pack": 0.0, "gram": 0.0, "rowsolve": 0.0,
            "finalize": 0.0, "rotate": 0.0, "unpack": 0.0}
    for layer in range(layers):
        for n, mods in groups.items():
            rows = sum(r for _, r in mods)
            nb = n // g
            work["syrk"] += float(N) * n * (n + 1)
            work["chol"] += n ** 3 / 3.0
            work["finalize"] += 28.0 * n * n       # rotated: S read twice (mirrored), T fp64 written and read, H fp32
            work["rotate"] += 8.0 * rows * n        # the weights' rotation: fp32 read and written
            work["sweep"] += rows * n * (4 + 1 + 2.0 / g) + n * n * 2.0
            for name, r in mods:
                b = _body.module_bits(layer, name, BODY["layers"])
                work["recode"] += r * n * (2 + 2.0 / g)
                work["pack"] += r * n * (1 + 2.0 / g) + r * n * b / 8.0 + r * n * 2.0 / g
                work["unpack"] += r * n * (1 + 2.0 / g) + r * n * b / 8.0 + r * n * 2.0 / g
            work["gram"] += 2 * 3.0 * rows * n * n                 # W'H + Gram, both joint solves
            work["rowsolve"] += 2 * rows * nb ** 3 / 3.0
    return work


def kernel_summary(db_path, steps, layers):
    """Markdown table of the library's kernels in a rocprofv3 kernel trace (rocpd database): calls,
    total and average duration, per-step time, and the roofline of the kernels whose algorithmic
    work per body step is stated (bf16 MFMA flops, fp64 flops, HBM bytes)."""
    import collections
    import re
    import sqlite3
    con = sqlite3.connect(db_path)
    cols = [r[1] for r in con.execute("pragma table_info(kernels)")]
    name_col = "name" if "name" in cols else "kernel_name"
    agg = collections.OrderedDict()
    busy, reach = 0.0, None  # time with at least one library kernel running (streams overlap)
    for name, start, end in con.execute(f"select {name_col}, start, end from kernels order by start"):
        m = re.search(r"wr::([A-Za-z0-9_]+(?:<[^>]*>)?)", name)
        if not m:
            continue
        a = agg.setdefault(m.group(1), [0, 0.0])
        a[0] += 1
        a[1] += (end - start) * 1e-3
        if reach is None or start >= reach:
            busy += (end - start) * 1e-3
            reach = end
        elif end > reach:
            busy += (end - reach) * 1e-3
            reach = end
    total = sum(v[1] for v in agg.values())
    out = [f"library kernels: {total / 1e3:.2f} ms of kernel time over {steps} step(s) = {total / 1e3 / steps:.2f} ms "
           f"per step; {busy / 1e3 / steps:.2f} ms per step with at least one of them running (kernels on "
           "different streams overlap, and then each one's duration includes the time it shares the chip)", "",
           "| kernel | calls | total ms | avg us | ms per step | share |", "|---|---|---|---|---|---|"]
    for k, (c, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        out.append(f"| `{k}` | {c} | {t / 1e3:.2f} | {t / c:.1f} | {t / 1e3 / steps:.2f} | {100 * t / total:.1f} % |")
    work = body_work(layers)
    kinds = [("syrk", r"^syrk_bf16_kernel|^syrk_reduce_kernel", "bf16 MFMA", PEAK_BF16_TFLOPS * 1e12, "TFLOP/s"),
             ("chol", r"^chol_", "fp64", 78.6e12, "TFLOP/s"),
             ("sweep", r"^sweep_panel_kernel|^trail_wide_kernel|^split_mt_kernel|^build_m_kernel", "HBM",
              PEAK_HBM_GBS * 1e9, "GB/s"),
             ("recode", r"^wring_prep_kernel", "HBM", PEAK_HBM_GBS * 1e9, "GB/s"),
             ("pack", r"^pack_vec_kernel|^pack_codes_kernel|^pack_scales_kernel", "HBM", PEAK_HBM_GBS * 1e9, "GB/s"),
             ("unpack", r"^unpack_vec_kernel|^unpack_codes_kernel|^unpack_scales_kernel", "HBM", PEAK_HBM_GBS * 1e9,
              "GB/s"),
             ("finalize", r"^rot_rows_sym_kernel|^rot_cols_damp_kernel", "HBM", PEAK_HBM_GBS * 1e9, "GB/s"),
             ("rotate", r"^fwht_rows", "HBM", PEAK_HBM_GBS * 1e9, "GB/s"),
             ("gram", r"^gram_lh_kernel|^rhs_sum_kernel", "bf16 MFMA", PEAK_BF16_TFLOPS * 1e12, "TFLOP/s"),
             ("rowsolve", r"^row_solve", "fp64", 78.6e12, "TFLOP/s")]
    out += ["", f"Rooflines per step ({layers} layers; algorithmic work as stated in the design notes):", "",
            "| step | kernels | bound | ms per step | achieved | peak | fraction |", "|---|---|---|---|---|---|---|"]
    for key, pat, bound, peak, unit in kinds:
        t = sum(v[1] for k, v in agg.items() if re.search(pat, k)) / steps
        if t <= 0:
            continue
        rate = work[key] / (t * 1e-6)
        scale = 1e12 if unit == "TFLOP/s" else 1e9
        out.append(f"| {key} | `{pat}` | {bound} | {t / 1e3:.2f} | {rate / scale:.1f} {unit} | "
                   f"{peak / scale:.0f} {unit} | {rate / peak:.3f} |")
    return "\n".join(out)


def main():
    args = parse()
    # before anything touches the GPU: HIP reads it once, when its runtime starts
    os.environ["GPU_MAX_HW_QUEUES"] = str(args.hw_queues)
    if args.kernel_summary:
        print(kernel_summary(args.kernel_summary, args.trace_steps, args.layers))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the solve runs on one GPU; --gpus must be 1 (across GPUs it would shard over "
              "calibration rows for H and over weight rows for the sweep and the wring)", file=sys.stderr)
        sys.exit(2)
    if args.syrk:
        main_syrk(args)
    elif args.workload == "q_proj":
        main_q_proj(args)
    else:
        main_body(args)


def main_syrk(args):
    """The H accumulation alone: S = X^T X over 262144 rows of input dim N (bf16, Gaussian; the
    kernel's time does not depend on the values), `steps` calls timed with HIP events."""
    import torch
    from post_bit_weight_amd import _lib as wr
    n, N = args.syrk, BODY["calib_rows"]
    ctx = wr.Context(0)
    gen = torch.Generator(device="cuda").manual_seed(20261203)
    X = torch.randn(N, n, device="cuda", generator=gen, dtype=torch.float32).to(torch.bfloat16)
    S = torch.empty(n, n, dtype=torch.float64, device="cuda")
    empty = torch.empty(0, n, dtype=torch.bfloat16, device="cuda")
    if args.copy_calibration > 0:
        src = torch.ones((args.copy_calibration << 20) // 4, dtype=torch.float32, device="cuda")
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    for _ in range(max(args.warmup, 0)):
        wr.wr_hessian_accumulate(ctx, X, S, zero=True)
    ts = []
    for _ in range(args.steps):
        wr.wr_hessian_accumulate(ctx, empty, S, zero=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(ctx.stream)
        wr.wr_hessian_accumulate(ctx, X, S)
        e1.record(ctx.stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = sum(ts) / len(ts)
    tf = float(N) * n * (n + 1) / (ms * 1e-3) / 1e12
    # the platform's GEMM (torch.mm, hipBLASLt) on the same operand layout for context: X^T X over
    # 16384-row chunks as a full square product (twice the useful flops)
    Xc = X[:16384]
    for _ in range(2):
        torch.mm(Xc.t(), Xc)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(N // 16384):
        torch.mm(Xc.t(), Xc)
    e1.record()
    torch.cuda.synchronize()
    mm_ms = e0.elapsed_time(e1)
    mm_tf = 2.0 * N * n * n / (mm_ms * 1e-3) / 1e12
    print(json.dumps({"syrk_n": n, "rows": N, "ms": ms, "tflops": tf, "frac": tf / PEAK_BF16_TFLOPS,
                      "torch_mm_full_square_ms": mm_ms, "torch_mm_tflops": mm_tf,
                      "torch_mm_frac": mm_tf / PEAK_BF16_TFLOPS}), flush=True)


if __name__ == "__main__":
    main()
