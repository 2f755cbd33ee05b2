"""Four-direction Hope memory scan on MI355X (gfx950): C-ABI HIP library + thin binding.

The scan itself lives in libhopescan.so (built by ``self_modifying_memory_amd.build``);
``self_modifying_memory_amd.scan2d`` marshals torch device tensors into its C ABI.
"""
from ._native import load_library, LIB_PATH, HEADER_PATH  # noqa: F401

__all__ = ["load_library", "LIB_PATH", "HEADER_PATH"]
