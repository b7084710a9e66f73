"""MI355X-native streaming-MoE decode step: HIP kernels behind a C ABI.

The hot path lives in ``csrc/`` (hand-written HIP for gfx950) and is exported
as a C-ABI shared library (``libsmd.so``); ``api`` is the thin ctypes binding
with the same entry-point names. ``synth`` holds the seeded input generators.
Importing this package does not load the library; ``api`` does, and raises if
it is missing.
"""
