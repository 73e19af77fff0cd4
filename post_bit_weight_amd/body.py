"""Quantize a whole Qwen3-4B-shaped transformer body, layer by layer, into one container.

Shapes and recipe (Wringer Qwen3-4B model card, "Recipe": 36 layers x 7 linears = 252 modules,
one GPTQ solve per layer on calibration rows, joint scales with lambda = 0.01, the wring, packed
codes plus fp16 block scales in one container):

* per layer, one H per input dimension: 2560 (q, k, v, gate, up), 4096 (o), 9728 (down), each
  accumulated from `calib_rows` calibration rows streamed in chunks of `chunk` rows;
* random-sign Hadamard rotation with blocks of 512 (which divides 2560, 4096 and 9728, so no
  padding): H is rotated in fp64 by wr_hessian_finalize and the weights by wr_hadamard_rotate;
* bit widths: 3 bits on v, o and down in every layer and on k in the first half of the layers,
  2 bits elsewhere, which gives 2.6396 bits per weight with fp16 scales on blocks of 64;
* a rank-128 adapter (alpha 128) per module drives the wring;
* every packed module is unpacked again on the device and compared with the codes and scales it
  was packed from (bit-exact round trip).

Inputs are seeded synthetic stand-ins for the pages' calibration corpus and checkpoint: the
calibration rows of layer l use the spectral model (product model for the 9728 input) with one
Haar basis per input dimension and per-layer draws; weights are Student-t (std 0.02); adapters
N(0, 0.01^2) in the rotated basis.

Every step of the solve runs in libwringer.so; this module only draws inputs, allocates device
memory and sequences the calls.  Run: python -m post_bit_weight_amd.body [--layers 36] [--out F]
"""

import argparse
import json
import os
import sys
import time

import torch

from . import _lib as wr
from . import measures, pipeline, synth

MODULES = [  # name, output rows, input dim
    ("q", 4096, 2560), ("k", 1024, 2560), ("v", 1024, 2560), ("gate", 9728, 2560), ("up", 9728, 2560),
    ("o", 2560, 4096), ("down", 2560, 9728),
]
DIMS = (2560, 4096, 9728)


def module_bits(layer, name, layers=36):
    if name in ("v", "o", "down"):
        return 3
    if name == "k" and layer < layers // 2:
        return 3
    return 2


def ledger(layers=36, group=64):
    """(weights, code bits, scale count) of the body for the bit mix above."""
    weights = code_bits = scales = 0
    for layer in range(layers):
        for name, rows, n in MODULES:
            weights += rows * n
            code_bits += rows * n * module_bits(layer, name, layers)
            scales += rows * (n // group)
    return weights, code_bits, scales


class CalibrationStream:
    """Chunks of calibration rows for one layer and input dim; chunk k of layer l is reproducible."""

    def __init__(self, n, base_seed, device):
        self.n = n
        self.src = synth.SpectralSource(n, seed=base_seed, device=device, outlier_frac=0.01, product=(n == 9728))
        self.base_seed = base_seed

    def chunk(self, layer, k, rows):
        self.src.seed = self.base_seed * 1009 + layer
        return self.src.chunk(k, rows)


class _Timer:
    """Sums the GPU time of the library calls only (HIP events on the library's stream), leaving out
    the drawing of synthetic inputs."""

    def __init__(self, stream):
        self.stream = stream
        self.pairs = []

    def start(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def stop(self, e0):
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record(self.stream)
        self.pairs.append((e0, e1))

    def total_ms(self):
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in self.pairs)


def quantize_layer(ctx, layer, streams, layers=36, calib_rows=262144, chunk=16384, had_block=512, group=64,
                   rank=128, seed=2026, keep=None, on_group=None, timer=None, measure=False):
    """One layer: returns {name: dict(packed (device uint8), rows, n, bits, roundtrip_ok[, measures])}.
    With measure, each module also gets the model cards' measures (measures.module_measures), computed
    after the layer's solve and outside the timer."""
    dev = ctx.device
    out = {}
    tick = timer.start if timer is not None else (lambda: None)
    tock = timer.stop if timer is not None else (lambda e: None)
    for n in DIMS:
        stream = streams[n]
        S = torch.empty(n, n, dtype=torch.float64, device=dev)
        total = 0
        for k in range(calib_rows // chunk):
            X = stream.chunk(layer, k, chunk)
            e = tick()
            wr.wr_hessian_accumulate(ctx, X, S, zero=(k == 0))
            tock(e)
            total += X.shape[0]
            del X
        signs = synth.signs(n, seed=seed * 7 + n, device=dev)
        raw = []
        for name, rows, dim in MODULES:
            if dim != n:
                continue
            ms = seed * 100003 + 1000 * layer + 10 * [m[0] for m in MODULES].index(name)
            raw.append((name, ms, synth.student_t((rows, n), seed=ms, device=dev, dtype=torch.bfloat16),
                        synth.gaussian((rows, rank), 0.01, seed=ms + 1, device=dev, dtype=torch.bfloat16),
                        synth.gaussian((rank, n), 0.01, seed=ms + 2, device=dev, dtype=torch.bfloat16)))
        e = tick()
        H, _ = pipeline.finalize_hessian(ctx, S, total, 0.01, n, had_block, signs)
        mods = []
        for name, ms, W, B, A in raw:
            mods.append(dict(name=name, bits=module_bits(layer, name, layers),
                             W=pipeline.prepare_weights(ctx, W, n, had_block, signs), W_raw=W, B=B, A=A,
                             alpha=float(rank)))
        res = pipeline.solve_group(ctx, mods, H, group, keep_stages=keep is not None or measure)
        tock(e)
        for m in mods:
            r = res[m["name"]]
            rows = m["W"].shape[0]
            c2 = torch.empty_like(r["codes"])
            s2 = torch.empty_like(r["scales"])
            wr.wr_unpack(ctx, r["packed"], rows, n, m["bits"], group, c2, s2)
            ok = bool(torch.equal(c2, r["codes"]) and torch.equal(s2.view(torch.int16), r["scales"].view(torch.int16)))
            out[m["name"]] = dict(packed=r["packed"], rows=rows, n=n, bits=m["bits"], roundtrip_ok=ok)
            if measure:
                bits_t = torch.full((rows,), m["bits"], dtype=torch.uint8, device=dev)
                out[m["name"]]["measures"] = measures.module_measures(
                    ctx, H, m["W"], bits_t, group, 0.01, r["gptq_codes"], r["joint_scales"], m["B"], m["A"], m["alpha"])
        if on_group is not None:
            on_group(n, dict(S=S, H=H, total=total, signs=signs, modules=mods, result=res, stream=stream))
        info = res["_dev_info"]
        if int(info.abs().sum().item()) != 0:
            raise RuntimeError(f"layer {layer}, input dim {n}: dev_info {info.tolist()}")
        del S, H, res, mods
    return out


def read_container(blob):
    """(entries {name: uint8 numpy array}, wringer_meta dict) of a container written by
    pipeline.container_bytes (an 8-byte little-endian header length, the JSON header, the blobs)."""
    import numpy as np
    hlen = int.from_bytes(blob[:8], "little")
    header = json.loads(bytes(blob[8:8 + hlen]))
    meta = json.loads(header.pop("__metadata__")["wringer_meta"])
    base = 8 + hlen
    entries = {}
    for name, spec in header.items():
        a, b = spec["data_offsets"]
        entries[name] = np.frombuffer(bytes(blob[base + a:base + b]), dtype=np.uint8)
    return entries, meta


def resumable_layers(meta, layers, group, had_block, rank):
    """Layers whose seven modules a previous container already holds with this body's shapes and bit
    mix (the state the pages' v0.3 re-finish starts from is the stored module, keyed by layer and
    module); raises if the container was made with another group, rotation block or rank."""
    for key, want in (("group", group), ("had_block", had_block), ("rank", rank)):
        if meta.get(key) != want:
            raise ValueError(f"container has {key} {meta.get(key)}, this run {want}")
    done = set()
    for layer in range(layers):
        ok = True
        for name, rows, n in MODULES:
            m = meta["modules"].get(f"layers.{layer}.{name}")
            if m != {"rows": rows, "n": n, "bits": module_bits(layer, name, layers)}:
                ok = False
                break
        if ok:
            done.add(layer)
    return done


def sweep_body(ctx, layers=36, calib_rows=262144, chunk=16384, had_block=512, group=64, rank=128, seed=2026,
               layer_ids=None, log=print, measure_layers=(), resume=None):
    """Quantize layers (all, or layer_ids) and build the container.  Returns (container bytes, report).
    resume: the bytes of an earlier container; the layers it holds completely are copied from it
    instead of solved again (report["resumed_layers"])."""
    dev = ctx.device
    streams = {n: CalibrationStream(n, seed * 31 + n, dev) for n in DIMS}
    entries, meta = [], {"format": "wringer", "group": group, "had_block": had_block, "rank": rank, "modules": {}}
    roundtrip = True
    measured = {}
    t0 = time.perf_counter()
    timer = _Timer(ctx.stream)
    ids = list(range(layers)) if layer_ids is None else list(layer_ids)
    old_entries, old_meta, done = {}, None, set()
    if resume is not None:
        old_entries, old_meta = read_container(resume)
        done = resumable_layers(old_meta, layers, group, had_block, rank)
    resumed = []
    for layer in ids:
        if layer in done:
            for name, _, _ in MODULES:
                key = f"layers.{layer}.{name}"
                entries.append((key + ".packed", old_entries[key + ".packed"]))
                meta["modules"][key] = old_meta["modules"][key]
            resumed.append(layer)
            log(f"layer {layer}: taken from the earlier container")
            continue
        res = quantize_layer(ctx, layer, streams, layers, calib_rows, chunk, had_block, group, rank, seed,
                             timer=timer, measure=layer in measure_layers)
        for name, r in res.items():
            key = f"layers.{layer}.{name}"
            entries.append((key + ".packed", r["packed"].cpu().numpy()))
            meta["modules"][key] = {"rows": r["rows"], "n": r["n"], "bits": r["bits"]}
            if "measures" in r:
                measured[key] = r["measures"]
            roundtrip &= r["roundtrip_ok"]
        log(f"layer {layer}: done ({time.perf_counter() - t0:.1f} s elapsed)")
    blob = pipeline.container_bytes(entries, meta)
    payload = sum(e[1].size for e in entries)
    weights = sum(v["rows"] * v["n"] for v in meta["modules"].values())
    report = {"layers": len(ids), "weights": weights, "payload_bytes": payload,
              "bits_per_weight": 8.0 * payload / weights, "container_bytes": len(blob),
              "roundtrip_bit_exact": roundtrip, "wall_s": time.perf_counter() - t0, "resumed_layers": resumed}
    if measured:
        report["measures"] = measured
    solve_ms = timer.total_ms()
    report["solve_gpu_ms"] = solve_ms
    solved = weights - sum(rows * n for _, rows, n in MODULES) * len(resumed)
    report["weights_per_s"] = solved / (solve_ms * 1e-3) if solve_ms > 0 else None
    return blob, report


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--layers", type=int, default=36)
    p.add_argument("--calib-rows", type=int, default=262144)
    p.add_argument("--out", default=None, help="write the container here")
    p.add_argument("--measure", default="", help="comma-separated layers whose modules also get the model cards' "
                                                  "measures (grid distance, solver disagreement, projection moves)")
    p.add_argument("--resume", default=None, help="an earlier container: its complete layers are kept, the rest solved")
    args = p.parse_args()
    ctx = wr.Context(0)
    ml = tuple(int(x) for x in args.measure.split(",") if x.strip())
    resume = open(args.resume, "rb").read() if args.resume else None
    blob, report = sweep_body(ctx, layers=args.layers, calib_rows=args.calib_rows,
                              log=lambda m: print(m, flush=True), measure_layers=ml, resume=resume)
    if args.out:
        with open(args.out, "wb") as f:
            f.write(blob)
    print(json.dumps(report), flush=True)
    if not report["roundtrip_bit_exact"]:
        sys.exit(1)


if __name__ == "__main__":
    main()
