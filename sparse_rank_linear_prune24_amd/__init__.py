"""2:4 sparse + rank-r linear layers on MI355X (gfx950).

The compute path is the HIP library `libsplr.so` (C ABI declared in include/splr.h); the Python
binding in `.binding` only marshals arguments to it.
"""
__all__ = ["configs", "inputs"]
