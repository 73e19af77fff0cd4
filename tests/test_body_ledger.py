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
