"""MI355X-native BitNet b1.58 BitLinear (W1.58A8) hot path.

The compute lives in ``libbitlinear.so`` (hand-written HIP kernels for gfx950
behind the C ABI declared in ``include/bitlinear.h``).  ``binding`` is a thin
ctypes layer over that ABI (it loads the library on first use and raises if
it was not built); ``layers`` holds BitLinear and BitNetFFN objects over it;
``synth`` draws the seeded synthetic inputs.
"""
from . import binding, layers, synth  # noqa: F401

__all__ = ["binding", "layers", "synth"]
