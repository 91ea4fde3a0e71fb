"""q4lin: the 4-bit quantized linear layer of a diffusion transformer on MI355X.

The compute lives in ``libq4lin.so`` (hand-written HIP for gfx950 behind a C ABI
declared in ``include/q4lin.h``).  ``binding`` is a thin ctypes layer that passes
device pointers, sizes and the current HIP stream; it raises if the library is not
built.  ``synth`` draws the seeded synthetic inputs.
"""

__all__ = ["binding", "synth"]
