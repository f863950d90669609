"""Tile-sparse video attention for AMD Instinct MI355X (gfx950).

The compute lives in libvsa.so (C ABI, include/vsa.h); `vsa` is its thin
ctypes binding. Importing this package loads nothing; the first call into
`vsa` loads the library and raises if it has not been built.
"""

__all__ = ["vsa"]
