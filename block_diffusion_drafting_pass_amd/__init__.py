"""MI355X-native DFlash block-diffusion draft pass.

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``, declared in ``include/dflash.h``); ``binding`` is a thin
ctypes layer over it that takes torch tensors for device memory and streams.
``inputs`` generates the seeded synthetic workloads.
"""
