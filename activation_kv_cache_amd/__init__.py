"""ByteCross decode step on MI355X (gfx950): activation-sparse projection GEMV
and split-K GQA decode attention over a dense or attention-selected KV cache.

The compute lives in libbc.so (HIP, include/bc.h); `binding` is its thin
ctypes binding, `inputs` the seeded synthetic input generators.  Importing
the package does not load the library; importing `binding` does, and fails
loudly when it is not built.
"""
__all__ = ["binding", "inputs"]
