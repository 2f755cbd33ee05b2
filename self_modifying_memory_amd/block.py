"""Python binding of the block C ABI (include/hope_block.h) over torch device tensors.

Argument marshalling only: every step of the block runs in the HIP kernels of
libhopescan.so (the projections, depthwise convolutions and norms in block_kernels.hip,
the operator in the scan kernels); torch supplies device memory and the stream.
"""
from __future__ import annotations

import ctypes

import torch

from . import _native as N
from .scan2d import HopeError, _check_numel, _keep_for_stream, _require_device

# weights whose entries are bf16 (passed as bit patterns)
_BF16_FIELDS = ("w_in", "w_q", "w_out", "w1", "w2")


def block_weight_numel(D: int, D_m: int, n_heads: int, ffn_dim: int) -> dict:
    """Elements of every weight of hope_block_weights_t for these sizes (the layouts the
    header documents); -1 where the head split is not an integer."""
    d = D_m // n_heads if n_heads > 0 and D_m % n_heads == 0 else -1
    S = 4 * d * d + 2 * d if d > 0 else -1
    return {"cpe_w": 9 * D, "cpe_b": D, "ln1_g": D, "ln1_b": D, "w_in": D_m * D, "b_in": D_m,
            "dw_w": 9 * D_m, "dw_b": D_m, "w_q": D_m * D_m,
            "init_memories": 4 * n_heads * S if S > 0 else -1, "route_scales": 4 * D_m,
            "skip": D_m, "lpe_w": 9 * D_m, "lpe_b": D_m, "w_out": D * D_m, "b_out": D,
            "ln2_g": D, "ln2_b": D, "w1": ffn_dim * D, "b1": ffn_dim, "w2": D * ffn_dim, "b2": D}


def hope_block_workspace_size(B: int, H: int, W: int, D: int, n_heads: int, ffn_dim: int,
                              chunk: int = 0, D_m: int | None = None) -> int:
    Dm = D if D_m is None else D_m
    return int(N.load_library().hope_block_workspace_size(B, H, W, D, Dm, n_heads, ffn_dim, chunk))


def hope_block_forward(x: torch.Tensor, weights: dict, n_heads: int, ffn_dim: int | None = None,
                       chunk: int = 0, *, D_m: int | None = None, out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One VisionHOPE block on x (fp32 [B, H, W, D], device).  weights: device tensors named
    as the fields of hope_block_weights_t (linear weights bf16 [out, in], the rest fp32).
    D_m: the operator's width (default D), split into n_heads heads; ffn_dim default 4 D."""
    lib = N.load_library()
    _require_device(x, "x")
    if x.dtype != torch.float32 or x.dim() != 4:
        raise ValueError("x must be fp32 [B, H, W, D]")
    B, H, W, D = x.shape
    F = 4 * D if ffn_dim is None else ffn_dim
    Dm = D if D_m is None else D_m
    numel = block_weight_numel(D, Dm, n_heads, F)
    wt = N.hope_block_weights_t()
    for name in N.BLOCK_WEIGHT_FIELDS:
        t = weights[name]
        _require_device(t, name)
        want = torch.bfloat16 if name in _BF16_FIELDS else torch.float32
        if t.dtype != want:
            raise ValueError(f"{name} must be {want}")
        _check_numel(t, numel[name], name)
        setattr(wt, name, t.data_ptr())
    if out is None:
        out = torch.empty_like(x)
        _keep_for_stream(out, stream)
    _require_device(out, "out")
    if out.dtype != torch.float32 or tuple(out.shape) != tuple(x.shape):
        raise ValueError("out must be fp32 shaped like x")
    need = hope_block_workspace_size(B, H, W, D, n_heads, F, chunk, Dm)
    if need == 0:
        raise HopeError(N.HOPE_ERR_INVALID_ARG, "hope_block_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        _keep_for_stream(workspace, stream)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    st = lib.hope_block_forward(x.data_ptr(), B, H, W, D, Dm, n_heads, F, chunk, ctypes.byref(wt),
                                out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                stream.cuda_stream)
    if st != N.HOPE_OK:
        raise HopeError(st, "hope_block_forward")
    return out
