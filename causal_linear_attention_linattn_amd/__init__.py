"""Causal linear attention for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI HIP library (liblinattn.so, built in this
directory); `ops` holds the thin Python binding.  `synth` is the seeded input
generator.  Importing this package does not load the library; the first call
into `ops` does, and raises if it is missing.
"""
__all__ = ["ops", "synth"]
