"""Hybrid sliding-window decode attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library `libhswd.so` (C ABI, `include/hswd.h`);
this package is a thin ctypes binding over it.  Torch tensors supply device
memory and the stream; every step of the decode path runs in the library's
kernels.  Calling an op when the library has not been built raises.
"""
