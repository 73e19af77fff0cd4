"""The 36-layer body driver on the GPU: two layers at their full per-layer size.

Layer 0 and layer 35 (different bit mixes: k is 3-bit in the first half of the body) are
quantized with 262144 calibration rows per H streamed in 16 chunks of 16384 rows, Hadamard
blocks of 512; every packed module must unpack bit-exactly, the container must parse back.  The
oracle checks layer 0's H for input dim 2560 (its own fp64 H from the same streamed rows, rotated
and damped), sampled entries of S for 4096 and 9728, and sampled rows through every stage, on the
GPU's H: q (2-bit), k (3-bit), v (3-bit), o (3-bit, 64 blocks) and down (3-bit, 152 blocks) of
layer 0, q and k (2-bit) of layer 35.
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


def _sampled_s_check(S_dev, stream, layer, n, rng, count=96):
    """Sampled entries of the accumulated S (lower triangle, fp64) against the oracle's sums of
    products over the same 16 streamed chunks of 16384 rows."""
    i = rng.integers(0, n, size=count)
    j = rng.integers(0, n, size=count)
    pairs = [(max(a, b), min(a, b)) for a, b in zip(i, j)] + [(k, k) for k in rng.integers(0, n, size=16)]
    cols = sorted({c for p in pairs for c in p})
    where = {c: t for t, c in enumerate(cols)}
    idx = torch.tensor(cols, device="cuda")
    Xc = np.concatenate([stream.chunk(layer, k, 16384)[:, idx].float().cpu().numpy() for k in range(16)])
    ref = oracle.sum_of_products(Xc, [(where[a], where[b]) for a, b in pairs])
    S = S_dev.cpu().numpy()
    got = np.array([S[a, b] for a, b in pairs])
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    _log(f"body: layer {layer}, input dim {n}: sampled S relative error {err:.2e}")
    assert err <= 1e-5


def _check_rows(grp, names, count, rng, layer):
    """Guided oracle on `count` sampled rows of each named module, on the GPU's H (fp64) and stored
    rotated weights; the proxy loss uses the undamped H (the GPU's H less the damping)."""
    Hg = grp["H"].cpu().double().numpy()
    n = Hg.shape[0]
    delta = 0.01 * np.trace(grp["S"].cpu().numpy()) / grp["total"] / n
    H0 = Hg - delta * np.eye(n)
    sd = grp["signs"].double().cpu().numpy()
    for mod in grp["modules"]:
        if mod["name"] not in names:
            continue
        rows = mod["W"].shape[0]
        sel = np.sort(rng.choice(rows, count, replace=False))
        t = torch.as_tensor(sel, device="cuda")
        W = oracle.rotate_rows(mod["W_raw"][t].double().cpu().numpy(), 512, sd)
        assert np.abs(mod["W"][t].double().cpu().numpy() - W).max() <= 1e-6 * np.abs(W).max()
        out = grp["result"][mod["name"]]
        gpu = {k: out[k][t] for k in ("gptq_codes", "gptq_scales", "joint_scales", "codes", "scales")}
        _log(f"body: layer {layer}: guided oracle on {count} rows of {mod['name']} ({mod['bits']}-bit, {n // 64} "
             "blocks)")
        guided_check(gpu, mod["W"][t].double().cpu().numpy(), Hg, H0, mod["bits"], 64, 0.01,
                     mod["B"][t].double().cpu().numpy(), mod["A"].double().cpu().numpy(), 128.0)


@pytest.mark.timeout(1200)
def test_body_two_layers_full_size():
    from post_bit_weight_amd import _lib as wr
    from post_bit_weight_amd import body, pipeline

    ctx = wr.Context(0)
    seen = {}

    def keep(n, grp):
        seen[n] = grp

    streams = {n: body.CalibrationStream(n, 2026 * 31 + n, ctx.device) for n in body.DIMS}
    _log("body: layer 0")
    res0 = body.quantize_layer(ctx, 0, streams, keep=True, on_group=keep)
    torch.cuda.synchronize()
    assert all(r["roundtrip_ok"] for r in res0.values())
    assert {k: r["bits"] for k, r in res0.items()} == {"q": 2, "k": 3, "v": 3, "gate": 2, "up": 2, "o": 3, "down": 3}
    # oracle H for the 2560 group from the same streamed rows, rotated with blocks of 512, damped
    _log("body: oracle H for layer 0, input dim 2560")
    chunks = (streams[2560].chunk(0, k, 16384).float().cpu().numpy() for k in range(16))
    sd = seen[2560]["signs"].double().cpu().numpy()
    H0 = oracle.rotate_sym(oracle.second_moment_chunks(chunks), 512, sd)
    H, _ = oracle.damp(H0, 0.01)
    Hg = seen[2560]["H"].cpu().double().numpy()
    err = np.linalg.norm(Hg - H) / np.linalg.norm(H)
    _log(f"body: H relative error {err:.2e}")
    assert err <= 1e-5
    rng = np.random.default_rng(11)
    _check_rows(seen[2560], ("q", "k", "v"), 4, rng, 0)
    for n, names in ((4096, ("o",)), (9728, ("down",))):
        _sampled_s_check(seen[n]["S"], streams[n], 0, n, rng)
        _check_rows(seen[n], names, 2, rng, 0)
    seen.clear()
    torch.cuda.empty_cache()
    _log("body: layer 35 (k is 2-bit in the second half of the layers)")

    def keep_2560(n, grp):
        if n == 2560:
            seen[n] = grp

    res35 = body.quantize_layer(ctx, 35, streams, keep=True, on_group=keep_2560)
    torch.cuda.synchronize()
    assert all(r["roundtrip_ok"] for r in res35.values())
    assert res35["k"]["bits"] == 2 and res35["q"]["bits"] == 2
    _check_rows(seen[2560], ("q", "k"), 3, rng, 35)
    seen.clear()
    del res0, res35
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
    # resume from that container: layers 0 and 35 are taken from it, layer 1 is solved
    _log("body: resume with layers 0, 35 stored and layer 1 to solve")
    blob2, rep2 = body.sweep_body(ctx, layer_ids=[0, 1, 35], log=_log, resume=blob)
    assert rep2["resumed_layers"] == [0, 35] and rep2["roundtrip_bit_exact"]
    back2 = st.load(blob2)
    assert len(back2) == 21
    for key, buf in back.items():
        assert np.array_equal(back2[key], buf)
    _log(f"body: {json.dumps(report)}")
