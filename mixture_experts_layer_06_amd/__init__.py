"""MI355X-native sparse MoE layer: HIP kernels for gfx950 behind a C ABI
(include/moe.h, libmoe.so), a ctypes binding (``binding``), the layer chain
(``layer``) and seeded synthetic workloads (``workloads``).

Importing the package does not load the HIP library; ``binding.load()`` does,
and raises if it has not been built.
"""
