"""ctypes view of libhopescan.so (the C ABI of include/hope_scan2d.h and include/hope_block.h).

Loading fails loudly when the library has not been built: there is no other
implementation of the scan in this package.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libhopescan.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "hope_scan2d.h")
BLOCK_HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "hope_block.h")

HOPE_OK = 0
HOPE_ERR_INVALID_ARG = -1
HOPE_ERR_UNSUPPORTED = -2
HOPE_ERR_WORKSPACE = -3
HOPE_ERR_HIP = -4

HOPE_F32 = 0
HOPE_BF16 = 1
HOPE_ETA_SIGMOID = 0
HOPE_ETA_SOFTPLUS = 1
HOPE_READOUT_BOUNDARY = 0
HOPE_READOUT_RUNNING = 1
HOPE_INJECTION = {"soft": 0, "hard": 1, "none": 2}
HOPE_SPECTRAL = {"clamp": 0, "soft": 1, "none": 2}
HOPE_FREEZE = {"kv": 1, "dynamics": 2, "q": 4}
HOPE_DIR_ALL = 15
HOPE_NOALLOC_SCRATCH_BYTES = 64 << 20


class hope_fmap_t(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("B", ctypes.c_int32),
                ("H", ctypes.c_int32), ("W", ctypes.c_int32), ("D", ctypes.c_int32),
                ("n_heads", ctypes.c_int32)]


class hope_scan2d_opts_t(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("final_memories", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("eta_map", ctypes.c_int32), ("eta_scale", ctypes.c_float),
                ("alpha_bias", ctypes.c_float), ("eps", ctypes.c_float),
                ("init_per_image", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("scan_begin", ctypes.c_void_p), ("scan_end", ctypes.c_void_p),
                ("readout", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("route_scales", ctypes.c_void_p), ("skip", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("injection", ctypes.c_int32),
                ("spectral", ctypes.c_int32), ("frozen", ctypes.c_uint32),
                ("no_dgd", ctypes.c_int32), ("shared_init", ctypes.c_int32),
                ("queries_dtype", ctypes.c_int32), ("queries", ctypes.c_void_p),
                ("mem_chunk", ctypes.c_int32), ("step_map", ctypes.c_void_p)]


BLOCK_WEIGHT_FIELDS = ("cpe_w", "cpe_b", "ln1_g", "ln1_b", "w_in", "b_in", "dw_w", "dw_b", "w_q",
                      "init_memories", "route_scales", "skip", "lpe_w", "lpe_b", "w_out", "b_out",
                      "ln2_g", "ln2_b", "w1", "b1", "w2", "b2")


class hope_block_weights_t(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in BLOCK_WEIGHT_FIELDS]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libhopescan.so once and declare every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m self_modifying_memory_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.hope_scan2d_default_opts.argtypes = [P(hope_scan2d_opts_t)]
    lib.hope_scan2d_default_opts.restype = None
    lib.hope_scan2d_forward.argtypes = [P(hope_fmap_t), ctypes.c_void_p, ctypes.c_uint32,
                                        ctypes.c_int32, ctypes.c_void_p, P(hope_scan2d_opts_t)]
    lib.hope_scan2d_forward.restype = ctypes.c_int
    lib.hope_scan2d_forward_noalloc.argtypes = [P(hope_fmap_t), ctypes.c_void_p, ctypes.c_uint32,
                                                ctypes.c_int32, ctypes.c_void_p, P(hope_scan2d_opts_t)]
    lib.hope_scan2d_forward_noalloc.restype = ctypes.c_int
    lib.hope_scan2d_workspace_size.argtypes = [P(hope_fmap_t), ctypes.c_uint32, ctypes.c_int32,
                                               P(hope_scan2d_opts_t)]
    lib.hope_scan2d_workspace_size.restype = ctypes.c_size_t
    lib.hope_scan2d_backward.argtypes = [P(hope_fmap_t), ctypes.c_void_p, ctypes.c_uint32,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, P(hope_scan2d_opts_t)]
    lib.hope_scan2d_backward.restype = ctypes.c_int
    lib.hope_scan2d_backward_workspace_size.argtypes = [P(hope_fmap_t), ctypes.c_uint32, ctypes.c_int32,
                                                        P(hope_scan2d_opts_t)]
    lib.hope_scan2d_backward_workspace_size.restype = ctypes.c_size_t
    lib.hope_scan2d_kernel_name.argtypes = [P(hope_fmap_t), ctypes.c_uint32, ctypes.c_int32,
                                            P(hope_scan2d_opts_t)]
    lib.hope_scan2d_kernel_name.restype = ctypes.c_char_p
    lib.hope_status_string.argtypes = [ctypes.c_int]
    lib.hope_status_string.restype = ctypes.c_char_p
    lib.hope_last_hip_error.argtypes = []
    lib.hope_last_hip_error.restype = ctypes.c_int
    lib.hope_debug_cross_scan.argtypes = [P(hope_fmap_t), ctypes.c_uint32, ctypes.c_void_p,
                                          ctypes.c_void_p]
    lib.hope_debug_cross_scan.restype = ctypes.c_int
    lib.hope_debug_cross_merge.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    lib.hope_debug_cross_merge.restype = ctypes.c_int
    lib.hope_block_workspace_size.argtypes = [ctypes.c_int32] * 8
    lib.hope_block_workspace_size.restype = ctypes.c_size_t
    lib.hope_block_forward.argtypes = [ctypes.c_void_p] + [ctypes.c_int32] * 8 + [
        P(hope_block_weights_t), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.hope_block_forward.restype = ctypes.c_int
    _lib = lib
    return lib


def header_functions(path: str | None = None) -> list[str]:
    """Names of the functions declared in the public header."""
    paths = [path] if path else [HEADER_PATH, BLOCK_HEADER_PATH]
    text = "".join(open(p).read() for p in paths)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(hope_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))
