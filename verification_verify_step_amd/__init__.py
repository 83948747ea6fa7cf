"""MI355X (gfx950) library of the speculative-decoding verify step.

``binding`` is the ctypes binding of the C ABI (include/vstep.h);
``runtime`` allocates the library's device buffers with PyTorch and keeps the
handles together.  The compute path is the HIP library only: importing the
runtime without the built ``libvstep.so`` raises.
"""
from . import binding  # noqa: F401
