"""Bit-packing of codes and fp16 scales (oracle, test infrastructure only).

Wringer model cards, "What is in this repo": the container holds packed codes
plus fp16 block scales.  The pages give no bit layout; the one used here:

* codes: per row, code j occupies bits [j b, (j + 1) b) of the row's bit
  stream, least significant bit first within little-endian bytes; a row is
  n b / 8 bytes (n a multiple of 8);
* scales: IEEE fp16 bit patterns, little-endian, row-major [rows][n / g];
* buffer = all code rows, then all scales.
"""

import numpy as np


def code_bytes_per_row(n, bits):
    if (n * bits) % 8 != 0:
        raise ValueError("n * bits must be a multiple of 8")
    return n * bits // 8


def packed_bytes(rows, n, bits, group):
    return rows * code_bytes_per_row(n, bits) + 2 * rows * (n // group)


def pack(codes, scales, bits, group):
    """Return the packed buffer (uint8) for codes (rows x n) and scales (rows x n/group)."""
    codes = np.asarray(codes, dtype=np.int64)
    rows, n = codes.shape
    if np.any((codes < 0) | (codes >= (1 << bits))):
        raise ValueError("code out of range")
    nbytes = code_bytes_per_row(n, bits)
    # bit (j*b + i) of the row stream is bit i of code j
    stream = ((codes[:, :, None] >> np.arange(bits)[None, None, :]) & 1).astype(np.uint8)
    stream = stream.reshape(rows, n * bits)
    code_part = np.packbits(stream, axis=1, bitorder="little")
    assert code_part.shape == (rows, nbytes)
    scale_part = np.asarray(scales, dtype=np.float64).astype("<f2").view(np.uint8).reshape(-1)
    return np.concatenate([code_part.reshape(-1), scale_part])


def unpack(buf, rows, n, bits, group):
    """Inverse of pack: returns (codes int64 rows x n, scales float64 rows x n/group)."""
    buf = np.asarray(buf, dtype=np.uint8).reshape(-1)
    if buf.shape[0] != packed_bytes(rows, n, bits, group):
        raise ValueError("buffer size does not match the layout")
    nbytes = code_bytes_per_row(n, bits)
    code_part = buf[: rows * nbytes].reshape(rows, nbytes)
    stream = np.unpackbits(code_part, axis=1, bitorder="little").reshape(rows, n, bits)
    codes = (stream.astype(np.int64) << np.arange(bits)[None, None, :]).sum(axis=2)
    scales = buf[rows * nbytes:].view("<f2").astype(np.float64).reshape(rows, n // group)
    return codes, scales
