"""MI355X (gfx950) per-linear-layer quantization solve: H accumulation, Hadamard rotation,
GPTQ/LDLQ sweep, joint fp16 scales and the wring, bit packing.

The compute lives in ``libwringer.so`` (HIP, C ABI declared in ``include/wringer.h``);
``_lib`` is its ctypes binding and ``pipeline`` sequences the calls for one module.
"""

from . import _lib  # noqa: F401
from ._lib import Context, load  # noqa: F401

__all__ = ["Context", "load"]
