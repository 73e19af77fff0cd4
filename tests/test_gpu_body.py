"""The 36-layer body driver on the GPU: two layers at their full per-layer size.

Layer 0 and layer 35 (different bit mixes: k is 3-bit in the first half of the body) are
quantized with 262144 calibration rows per H streamed in 16 chunks of 16384 rows, Hadamard
blocks of 512; every packed module must unpack bit-exactly, the container must parse back, and
for layer 0's 2560-input group the oracle checks H (its own fp64 H from the same streamed rows,
rotated and damped) and sampled rows of q (2-bit), k (3-bit) and v (3-bit) through every stage.
"""
import json
import time

import numpy as np
import pytest
import torch

import oracle
from parity import guided_check

pytestmark = pytest.mark.gpu


def _log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def test_body_two_layers_full_size():
    from post_bit_weight_amd import _lib as wr
    from post_bit_weight_amd import body, pipeline

    ctx = wr.Context(0)
    seen = {}

    def keep_2560(n, grp):
        if n == 2560:
            seen.update(grp)

    streams = {n: body.CalibrationStream(n, 2026 * 31 + n, ctx.device) for n in body.DIMS}
    _log("body: layer 0")
    res0 = body.quantize_layer(ctx, 0, streams, keep=True, on_group=keep_2560)
    torch.cuda.synchronize()
    assert all(r["roundtrip_ok"] for r in res0.values())
    assert {k: r["bits"] for k, r in res0.items()} == {"q": 2, "k": 3, "v": 3, "gate": 2, "up": 2, "o": 3, "down": 3}
    # oracle H for the 2560 group from the same streamed rows, rotated with blocks of 512, damped
    _log("body: oracle H for layer 0, input dim 2560")
    chunks = (streams[2560].chunk(0, k, 16384).float().cpu().numpy() for k in range(16))
    sd = seen["signs"].double().cpu().numpy()
    H0 = oracle.rotate_sym(oracle.second_moment_chunks(chunks), 512, sd)
    H, _ = oracle.damp(H0, 0.01)
    Hg = seen["H"].cpu().double().numpy()
    err = np.linalg.norm(Hg - H) / np.linalg.norm(H)
    _log(f"body: H relative error {err:.2e}")
    assert err <= 1e-5
    rng = np.random.default_rng(11)
    for mod in seen["modules"]:
        if mod["name"] not in ("q", "k", "v"):
            continue
        rows = mod["W"].shape[0]
        sel = np.sort(rng.choice(rows, 4, replace=False))
        t = torch.as_tensor(sel, device="cuda")
        W = oracle.rotate_rows(mod["W_raw"][t].double().cpu().numpy(), 512, sd)
        assert np.abs(mod["W"][t].double().cpu().numpy() - W).max() <= 1e-6 * np.abs(W).max()
        out = seen["result"][mod["name"]]
        gpu = {k: out[k][t] for k in ("gptq_codes", "gptq_scales", "joint_scales", "codes", "scales")}
        _log(f"body: guided oracle on 4 rows of {mod['name']} ({mod['bits']}-bit)")
        guided_check(gpu, W, H, H0, mod["bits"], 64, 0.01, mod["B"][t].double().cpu().numpy(),
                     mod["A"].double().cpu().numpy(), 128.0, 2e-2)
    del seen
    torch.cuda.empty_cache()
    _log("body: layers 0 and 35 through the body driver, container")
    blob, report = body.sweep_body(ctx, layer_ids=[0, 35], log=_log)
    assert report["roundtrip_bit_exact"]
    w2, c2, s2 = 0, 0, 0
    for layer in (0, 35):
        for name, rows, n in body.MODULES:
            w2 += rows * n
            c2 += rows * n * body.module_bits(layer, name)
            s2 += rows * (n // 64)
    assert report["weights"] == w2 and report["payload_bytes"] == (c2 + 16 * s2) // 8
    st = pytest.importorskip("safetensors.numpy")
    back = st.load(blob)
    assert len(back) == 14
    hlen = int.from_bytes(blob[:8], "little")
    meta = json.loads(json.loads(blob[8:8 + hlen])["__metadata__"]["wringer_meta"])
    assert meta["modules"]["layers.0.k"]["bits"] == 3 and meta["modules"]["layers.35.k"]["bits"] == 2
    _log(f"body: {json.dumps(report)}")
