"""The container writer: safetensors-format bytes that an independent reader parses back."""
import json

import numpy as np
import pytest

from post_bit_weight_amd.pipeline import container_bytes


def test_container_round_trips_through_safetensors():
    st = pytest.importorskip("safetensors.numpy")
    rng = np.random.default_rng(3)
    a = rng.integers(0, 256, size=37, dtype=np.uint8)
    b = rng.integers(0, 256, size=1000, dtype=np.uint8)
    meta = {"format": "wringer", "modules": {"l0.q": {"bits": 2, "group": 64}}}
    blob = container_bytes([("l0.q.packed", a), ("l0.down.packed", b)], meta)
    got = st.load(blob)
    assert np.array_equal(got["l0.q.packed"], a) and np.array_equal(got["l0.down.packed"], b)
    hlen = int.from_bytes(blob[:8], "little")
    header = json.loads(blob[8:8 + hlen])
    assert json.loads(header["__metadata__"]["wringer_meta"]) == meta
    assert len(blob) == 8 + hlen + a.size + b.size and hlen % 8 == 0
