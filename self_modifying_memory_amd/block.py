"""Python binding of the block C ABI (include/hope_block.h) over torch device tensors.

Argument marshalling only: every step of the block runs in the HIP kernels of
libhopescan.so (the projections, depthwise convolutions and norms in block_kernels.hip,
the operator in the scan kernels); torch supplies device memory and the stream.
"""
from __future__ import annotations

import ctypes

import torch

from . import _native as N
from .scan2d import HopeError, _require_device

# weights whose entries are bf16 (passed as bit patterns)
_BF16_FIELDS = ("w_in", "w_q", "w_out", "w1", "w2")


def hope_block_workspace_size(B: int, H: int, W: int, D: int, n_heads: int, ffn_dim: int,
                              chunk: int = 0) -> int:
    return int(N.load_library().hope_block_workspace_size(B, H, W, D, n_heads, ffn_dim, chunk))


def hope_block_forward(x: torch.Tensor, weights: dict, n_heads: int, ffn_dim: int | None = None,
                       chunk: int = 0, *, out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One VisionHOPE block on x (fp32 [B, H, W, D], device).  weights: device tensors named
    as the fields of hope_block_weights_t (linear weights bf16 [out, in], the rest fp32)."""
    lib = N.load_library()
    _require_device(x, "x")
    if x.dtype != torch.float32 or x.dim() != 4:
        raise ValueError("x must be fp32 [B, H, W, D]")
    B, H, W, D = x.shape
    F = 4 * D if ffn_dim is None else ffn_dim
    wt = N.hope_block_weights_t()
    for name in N.BLOCK_WEIGHT_FIELDS:
        t = weights[name]
        _require_device(t, name)
        want = torch.bfloat16 if name in _BF16_FIELDS else torch.float32
        if t.dtype != want:
            raise ValueError(f"{name} must be {want}")
        setattr(wt, name, t.data_ptr())
    if out is None:
        out = torch.empty_like(x)
    _require_device(out, "out")
    need = hope_block_workspace_size(B, H, W, D, n_heads, F, chunk)
    if need == 0:
        raise HopeError(N.HOPE_ERR_INVALID_ARG, "hope_block_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    st = lib.hope_block_forward(x.data_ptr(), B, H, W, D, n_heads, F, chunk, ctypes.byref(wt),
                                out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                stream.cuda_stream)
    if st != N.HOPE_OK:
        raise HopeError(st, "hope_block_forward")
    return out
