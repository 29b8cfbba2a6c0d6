"""Spava / APB-V approximate-attention prefill on MI355X (gfx950).

The HIP library is reached through ``long_context_approximate_amd.spava`` (ctypes
binding over the C ABI declared in ``include/spava.h``). Importing this package does
not load the library.
"""
__all__ = ["inputs", "spava"]
