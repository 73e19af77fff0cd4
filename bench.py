"""Throughput of the whole per-module quantization solve on one MI355X.

One step = H accumulation over all calibration rows + finalize/damping + GPTQ
sweep + joint scales + wring (rank-128 adapter, nearest-point recode, joint
scales) + packing, for a Qwen3-4B-shaped q_proj (W 4096 x 2560 bf16, X
131072 x 2560 bf16, 2-bit, group 64, lazy batch 128, lambda 0.01).  Inputs are
synthetic and resident in HBM before the timed region.  The metric is weights
quantized per second.

Also reported: the roofline of the dominant kernel (the bf16 SYRK that
accumulates H: N n (n + 1) useful flops per call, timed live with HIP events on
the stream it runs on) and the CPU oracle timed on a bounded sample of the same
workload on the host cores, and, outside the timed step, the materializer (packed
module -> bf16 weights) against the HBM peak, the finisher variant with GPTQ
codes (wring by a GPTQ sweep of the watered target instead of nearest-point
codes), the trellis-coded quantizer (Viterbi search) against the VALU peak, and
the packed-module product (decode-time GEMV from the container) against the HBM
peak.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras | --extras-only]
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
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=128, help="weight rows in the oracle sample")
    p.add_argument("--cpu-calib", type=int, default=8192, help="calibration rows in the oracle sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="before the warmup, copy MIB mebibytes device to device once (a plain copy kernel of known "
                        "size, the yardstick for the FETCH_SIZE / WRITE_SIZE counters)")
    p.add_argument("--no-extras", action="store_true",
                   help="time the solve step only (no materializer or finisher-variant timing)")
    p.add_argument("--extras-only", action="store_true",
                   help="one untimed step (for H), then only the materializer and the finisher-variant timings")
    return p.parse_args()


def traffic_from_profile():
    """HBM bytes per SYRK launch from the committed rocprofv3 counter summary, if it matches this source.

    The summary holds `bytes_per_launch:` (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the
    counter reads for a plain 512 MiB copy) and `source_sha256:` of the kernel source it was taken on; once
    the source has changed the figure no longer describes the kernel and None is returned.
    """
    path = os.path.join(ROOT, "profiles", "syrk_bf16_q_proj_traffic.txt")
    src = os.path.join(ROOT, "post_bit_weight_amd", "csrc", "k_hessian.hip")
    try:
        rec = {}
        for line in open(path):
            if ":" in line and not line.startswith((" ", "#")):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if rec.get("source_sha256") != digest:
            return None
        return float(rec["bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def cpu_baseline(X_host, W_host, B_host, A_host, cfg, n_rows, n_calib):
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


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the solve runs on one GPU; --gpus must be 1 (across GPUs it would shard over "
              "calibration rows for H and over weight rows for the sweep and the wring)", file=sys.stderr)
        sys.exit(2)
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
    traffic = traffic_from_profile()
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
        line["cpu_baseline"] = cpu_baseline(Xh, Wh, Bh, Ah, cfg, args.cpu_rows, args.cpu_calib)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
