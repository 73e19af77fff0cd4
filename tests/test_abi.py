"""CPU checks of the C ABI: the header's declarations, the built library's exports, host-side paths."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wringer.h")
LIB = os.path.join(ROOT, "post_bit_weight_amd", "libwringer.so")


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(wr_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_names():
    from post_bit_weight_amd import _lib
    assert declared() == sorted(_lib.EXPORTED)


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    syms = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    missing = [s for s in declared() if s not in syms]
    assert not missing


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_library_loads_and_host_only_paths_work():
    from post_bit_weight_amd import _lib
    lib = _lib.load()
    assert lib.wr_strerror(0) == b"success"
    assert lib.wr_strerror(1) == b"invalid argument"
    # workspace sizing is pure host arithmetic
    ws = _lib.wr_workspace_bytes(_lib.WR_OP_GPTQ, 4096, 2560, 64, 0, 128)
    assert ws >= 2 * 2560 * 2560 * 4 + 4096 * 2560 * 4
    assert _lib.wr_workspace_bytes(_lib.WR_OP_WRING, 256, 512, 32, 8, 0) > 0
    assert _lib.wr_workspace_bytes(_lib.WR_OP_ROTATE, 8, 8, 0, 0, 0) == 0
    # argument errors are caught before any device call
    P = ctypes.c_void_p
    assert lib.wr_destroy(None) == _lib.WR_EINVAL
    assert lib.wr_create(None, 0, None) == _lib.WR_EINVAL
    assert lib.wr_hessian_accumulate(None, None, 1, 0, 8, 8, None, 0) == _lib.WR_EINVAL
    assert lib.wr_pack(None, None, None, 1, 8, 2, 8, None, 0) == _lib.WR_EINVAL
    assert lib.wr_set_workspace(None, None, 0) == _lib.WR_EINVAL


def test_missing_library_fails_loudly(tmp_path):
    from post_bit_weight_amd import _lib
    with pytest.raises(ImportError):
        _lib._open(str(tmp_path / "libwringer.so"))
