"""The body's bit mix reaches the ledger stated for the 36-layer workload (host arithmetic only)."""
import oracle
from post_bit_weight_amd import body


def test_body_bit_mix_ledger():
    weights, code_bits, scales = body.ledger(36)
    assert weights == 3633315840                      # 36 x (the seven Qwen3-4B-shaped linears)
    bpw, code, scale = oracle.ledger_bits_per_weight(weights, code_bits, scales)
    assert abs(bpw - 2.6396) < 1e-4                   # about 2.64 b/w including fp16 block scales
    payload = (code_bits + 16 * scales) // 8
    assert payload == 1198817280                      # 1.1165 GiB of packed codes and scales
    assert abs(payload / 2 ** 30 - 1.1165) < 1e-4


def test_container_reads_back_and_resume_finds_complete_layers():
    """Host-side resume logic: a container holding all seven modules of layer 0 and five of layer 1
    resumes layer 0 only; a container made with another group is refused."""
    import numpy as np
    import pytest
    from post_bit_weight_amd import pipeline
    entries, meta = [], {"format": "wringer", "group": 64, "had_block": 512, "rank": 128, "modules": {}}
    rng = np.random.default_rng(3)
    for layer, names in ((0, [m[0] for m in body.MODULES]), (1, ["q", "k", "v", "o", "down"])):
        for name, rows, n in body.MODULES:
            if name not in names:
                continue
            key = f"layers.{layer}.{name}"
            buf = rng.integers(0, 256, size=rows // 64 + 7, dtype=np.uint8)
            entries.append((key + ".packed", buf))
            meta["modules"][key] = {"rows": rows, "n": n, "bits": body.module_bits(layer, name)}
    blob = pipeline.container_bytes(entries, meta)
    back, meta2 = body.read_container(blob)
    assert meta2 == meta and set(back) == {e[0] for e in entries}
    for name, buf in entries:
        assert np.array_equal(back[name], buf)
    assert body.resumable_layers(meta2, 36, 64, 512, 128) == {0}
    with pytest.raises(ValueError):
        body.resumable_layers(meta2, 36, 32, 512, 128)
