"""Reduced Matrix Multiplication (RMM) hot path for AMD Instinct MI355X (gfx950).

The compute lives in librmm.so (hand-written HIP kernels behind a C ABI,
declared in include/rmm.h); `rmm` is its thin ctypes binding and `synth` the
seeded input generator.  Importing this package loads nothing: the library is
opened on first use by `rmm`, which raises if it has not been built.
"""
__all__ = ["rmm", "synth"]
