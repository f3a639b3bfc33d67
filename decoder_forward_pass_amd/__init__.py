"""Decoder forward pass on one AMD MI355X (gfx950): HIP kernels behind a C ABI.

The library ``libdec.so`` (built from ``csrc/`` by ``build.py``) implements the
C ABI of ``include/dec.h``: dec_init, dec_prefill, dec_decode_step, dec_free and
their layout/validation helpers. ``binding`` wraps it with ctypes under the
same names; ``session`` allocates the device buffers with torch and keeps a
host block allocator. Importing ``binding`` fails if the library is not built:
there is no fallback path.
"""

__all__ = ["binding", "blob", "session"]
