"""MI355X-native BitNet b1.58 BitLinear (W1.58A8) hot path.

The compute lives in ``libbitlinear.so`` (hand-written HIP kernels for gfx950
behind a C ABI declared in ``include/bitlinear.h``).  ``binding`` is a thin
ctypes layer over that ABI; ``synth`` draws the seeded synthetic inputs.
"""
from . import synth  # noqa: F401

__all__ = ["synth", "binding"]


def __getattr__(name):
    if name == "binding":
        from . import binding
        return binding
    raise AttributeError(name)
