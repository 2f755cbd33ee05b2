"""Python binding of the C ABI over torch device tensors.

Argument marshalling only: every step of the scan runs in the HIP kernels of
libhopescan.so.  torch supplies device memory and the stream.  Function names
follow include/hope_scan2d.h.
"""
from __future__ import annotations

import ctypes

import torch

from . import _native as N

_ETA_MAPS = {"sigmoid": N.HOPE_ETA_SIGMOID, "softplus": N.HOPE_ETA_SOFTPLUS}
_READOUTS = {"boundary": N.HOPE_READOUT_BOUNDARY, "running": N.HOPE_READOUT_RUNNING}


class HopeError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = N.load_library()
        name = lib.hope_status_string(status).decode()
        extra = f" (hipError {lib.hope_last_hip_error()})" if status == N.HOPE_ERR_HIP else ""
        super().__init__(f"{where}: {name}{extra}")
        self.status = status


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return N.HOPE_F32
    if t.dtype == torch.bfloat16:
        return N.HOPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _require_device(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _keep_for_stream(t: torch.Tensor | None, stream) -> None:
    """Tell torch's caching allocator that a tensor this wrapper allocated is used by the
    work enqueued on ``stream``: without it, the memory could be handed to a later
    allocation on the current stream while the kernels still write it."""
    if t is not None and stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)


def state_numel(x: torch.Tensor, n_heads: int, init_per_image: bool = False,
                shared_init: bool = False) -> int:
    """Elements of an initial-state tensor for x: S = 4d^2 + 2d floats per (route, head),
    times 4 routes (1 with shared_init), times B with init_per_image."""
    D = x.shape[3]
    if n_heads <= 0 or D % n_heads:
        return -1
    d = D // n_heads
    S = 4 * d * d + 2 * d
    return (x.shape[0] if init_per_image else 1) * (1 if shared_init else 4) * n_heads * S


def _check_numel(t: torch.Tensor, want: int, name: str) -> None:
    # a short buffer would be read or written out of bounds on the device: the C ABI
    # sees only pointers, so sizes are checked here, before the call
    if want >= 0 and t.numel() != want:
        raise ValueError(f"{name} must have {want} elements, has {t.numel()}")


def make_fmap(x: torch.Tensor, n_heads: int) -> N.hope_fmap_t:
    if x.dim() != 4:
        raise ValueError("x must be [B, H, W, D]")
    B, H, W, D = x.shape
    return N.hope_fmap_t(x.data_ptr(), _dtype_code(x), B, H, W, D, n_heads)


def make_opts(stream=None, eta_map: str = "sigmoid", eta_scale: float = 1.0,
              alpha_bias: float = 4.0, eps: float = 1e-6, init_per_image: bool = False,
              final_memories: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None,
              out_dtype: torch.dtype = torch.float32,
              readout: str = "boundary", variants: dict | None = None) -> N.hope_scan2d_opts_t:
    lib = N.load_library()
    o = N.hope_scan2d_opts_t()
    lib.hope_scan2d_default_opts(ctypes.byref(o))
    o.stream = _stream_handle(stream)
    o.eta_map = _ETA_MAPS[eta_map]
    o.eta_scale = eta_scale
    o.alpha_bias = alpha_bias
    o.eps = eps
    o.init_per_image = int(bool(init_per_image))
    o.out_dtype = N.HOPE_BF16 if out_dtype == torch.bfloat16 else N.HOPE_F32
    o.readout = _READOUTS[readout]
    _set_variants(o, variants or {})
    if final_memories is not None:
        _require_device(final_memories, "final_memories")
        if final_memories.dtype != torch.float32:
            raise TypeError("final_memories must be float32")
        o.final_memories = final_memories.data_ptr()
    if workspace is not None:
        _require_device(workspace, "workspace")
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel() * workspace.element_size()
    return o


def _f32_device(t: torch.Tensor, name: str, numel: int, check_device: bool = True) -> int:
    if check_device:
        _require_device(t, name)
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != numel:
        raise ValueError(f"{name} must be a contiguous float32 tensor of {numel} elements")
    return t.data_ptr()


def _set_variants(o: N.hope_scan2d_opts_t, v: dict, check_device: bool = True) -> None:
    """VisionHOPE variants (Eq. 26 scales, App. B.5 skip, Sec. 3.5 ablations)."""
    req = _require_device if check_device else (lambda t, name: None)
    unknown = set(v) - {"route_scales", "skip", "counts", "injection", "spectral", "frozen",
                        "no_dgd", "shared_init", "queries", "mem_chunk", "step_map", "n_heads",
                        "shape", "D"}
    if unknown:
        raise ValueError(f"unknown variant options {sorted(unknown)}")
    D = v.get("D")
    if v.get("route_scales") is not None:
        o.route_scales = _f32_device(v["route_scales"], "route_scales", 4 * D, check_device)
    if v.get("skip") is not None:
        o.skip = _f32_device(v["skip"], "skip", D, check_device)
    if v.get("counts") is not None:
        c = v["counts"]
        req(c, "counts")
        if c.dtype != torch.int64 or not c.is_contiguous() or c.numel() != 3:
            raise ValueError("counts must be a contiguous int64 tensor of 3 elements")
        o.counts = c.data_ptr()
    o.injection = N.HOPE_INJECTION[v.get("injection", "soft")]
    o.spectral = N.HOPE_SPECTRAL[v.get("spectral", "clamp")]
    o.frozen = sum(N.HOPE_FREEZE[f] for f in set(v.get("frozen", ())))
    o.no_dgd = int(bool(v.get("no_dgd", False)))
    o.shared_init = int(bool(v.get("shared_init", False)))
    q = v.get("queries")
    if q is not None:
        req(q, "queries")
        if q.dtype not in (torch.float32, torch.bfloat16) or not q.is_contiguous() or \
                tuple(q.shape) != tuple(v["shape"]):
            raise ValueError("queries must be a contiguous float32 / bfloat16 tensor shaped like x")
        o.queries = q.data_ptr()
        o.queries_dtype = N.HOPE_BF16 if q.dtype == torch.bfloat16 else N.HOPE_F32
    o.mem_chunk = int(v.get("mem_chunk", 0))
    sm = v.get("step_map")
    if sm is not None:
        B, H, W, _ = v["shape"]
        req(sm, "step_map")
        if sm.dtype != torch.float32 or not sm.is_contiguous() or sm.numel() != B * 4 * v["n_heads"] * H * W:
            raise ValueError("step_map must be a contiguous float32 tensor [B, 4, n_heads, H, W]")
        o.step_map = sm.data_ptr()


def hope_scan2d_kernel_name(x: torch.Tensor, n_heads: int, dirs: int = 15, chunk: int = 0,
                            readout: str = "boundary", out_dtype: torch.dtype = torch.float32,
                            **variants) -> str:
    """Name of the scan kernel hope_scan2d_forward launches for these arguments ("" when
    it would reject them).  Only shapes, dtypes and option flags are read; variant
    tensors may be given as in hope_scan2d_forward (their pointers are not dereferenced)."""
    lib = N.load_library()
    fm = make_fmap(x, n_heads)
    o = N.hope_scan2d_opts_t()
    lib.hope_scan2d_default_opts(ctypes.byref(o))
    o.out_dtype = N.HOPE_BF16 if out_dtype == torch.bfloat16 else N.HOPE_F32
    o.readout = _READOUTS[readout]
    v = dict(variants)
    v.update(n_heads=n_heads, shape=tuple(x.shape), D=x.shape[3])
    _set_variants(o, v, check_device=False)
    return lib.hope_scan2d_kernel_name(ctypes.byref(fm), dirs, chunk, ctypes.byref(o)).decode()


def hope_scan2d_workspace_size(x: torch.Tensor, n_heads: int, dirs: int = 15, chunk: int = 0,
                               out_dtype: torch.dtype = torch.float32) -> int:
    lib = N.load_library()
    fm = make_fmap(x, n_heads)
    o = N.hope_scan2d_opts_t()
    lib.hope_scan2d_default_opts(ctypes.byref(o))
    o.out_dtype = N.HOPE_BF16 if out_dtype == torch.bfloat16 else N.HOPE_F32
    return int(lib.hope_scan2d_workspace_size(ctypes.byref(fm), dirs, chunk, ctypes.byref(o)))


def alloc_workspace(x: torch.Tensor, n_heads: int, dirs: int = 15, chunk: int = 0,
                    out_dtype: torch.dtype = torch.float32) -> torch.Tensor | None:
    """A workspace of the size the library asks for (None when none is needed)."""
    nbytes = hope_scan2d_workspace_size(x, n_heads, dirs, chunk, out_dtype)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=x.device)


def hope_scan2d_forward(x: torch.Tensor, init_memories: torch.Tensor, n_heads: int, dirs: int = 15,
                        chunk: int = 0, out: torch.Tensor | None = None, *, stream=None,
                        eta_map: str = "sigmoid", eta_scale: float = 1.0, alpha_bias: float = 4.0,
                        eps: float = 1e-6, init_per_image: bool = False,
                        final_memories: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None,
                        scan_events: tuple | None = None,
                        readout: str = "boundary", route_scales: torch.Tensor | None = None,
                        skip: torch.Tensor | None = None, counts: torch.Tensor | None = None,
                        injection: str = "soft", spectral: str = "clamp", frozen=(),
                        no_dgd: bool = False, shared_init: bool = False,
                        queries: torch.Tensor | None = None, mem_chunk: int = 0,
                        step_map: torch.Tensor | None = None, _noalloc: bool = False) -> torch.Tensor:
    """Run the four-direction scan; returns ``out`` ([B, H, W, D] float32, or bfloat16
    when a bfloat16 ``out`` is passed: the fp32 route sum rounded once).

    init_memories: float32 [4, n_heads, 4d^2+2d] (or [B, 4, n_heads, ...] with
    init_per_image).  A workspace is allocated through torch when none is given.
    readout: "boundary" (memory frozen at the chunk start) or "running" (memory after
    the chunk's earlier tokens).
    Variants: route_scales [4, D] and skip [D] float32 (Eq. 26, App. B.5); counts, an int64
    [3] tensor the step-control counters are added to; injection "soft"/"hard"/"none";
    spectral "clamp"/"soft"/"none"; frozen, a subset of {"kv", "dynamics", "q"}; no_dgd;
    shared_init (init_memories is then [n_heads, S]); queries, a [B, H, W, D] tensor of
    queries from a fixed outer projection (M_q is then unused); mem_chunk > 0, the working
    memory's own chunk length (two chunk sizes; 0 = one length for all six memories);
    step_map, a float32 [B, 4, n_heads, H, W] tensor that receives the executed step of every
    token of a selected route at its pixel.
    scan_events: optional (begin, end) torch.cuda.Event pair that the library records
    around the scan kernel alone (already recorded once, so that they exist).
    """
    lib = N.load_library()
    _require_device(x, "x")
    _require_device(init_memories, "init_memories")
    if init_memories.dtype != torch.float32:
        raise TypeError("init_memories must be float32")
    _check_numel(init_memories, state_numel(x, n_heads, init_per_image, shared_init), "init_memories")
    if final_memories is not None:
        _check_numel(final_memories, state_numel(x, n_heads, True), "final_memories")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
        _keep_for_stream(out, stream)
    _require_device(out, "out")
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != tuple(x.shape):
        raise ValueError("out must be float32 or bfloat16 with the shape of x")
    if workspace is None and not _noalloc:
        workspace = alloc_workspace(x, n_heads, dirs, chunk, out.dtype)
        _keep_for_stream(workspace, stream)
    fm = make_fmap(x, n_heads)
    variants = dict(route_scales=route_scales, skip=skip, counts=counts, injection=injection,
                    spectral=spectral, frozen=frozen, no_dgd=no_dgd, shared_init=shared_init,
                    queries=queries, mem_chunk=mem_chunk, step_map=step_map, n_heads=n_heads,
                    shape=tuple(x.shape), D=x.shape[3])
    opts = make_opts(stream, eta_map, eta_scale, alpha_bias, eps, init_per_image, final_memories,
                     workspace, out.dtype, readout, variants)
    if scan_events is not None:
        begin, end = scan_events
        if not begin.cuda_event or not end.cuda_event:
            raise ValueError("scan_events must have been recorded once before use")
        opts.scan_begin, opts.scan_end = begin.cuda_event, end.cuda_event
    entry = lib.hope_scan2d_forward_noalloc if _noalloc else lib.hope_scan2d_forward
    st = entry(ctypes.byref(fm), init_memories.data_ptr(), dirs, chunk, out.data_ptr(), ctypes.byref(opts))
    if st != N.HOPE_OK:
        raise HopeError(st, "hope_scan2d_forward_noalloc" if _noalloc else "hope_scan2d_forward")
    return out


def hope_scan2d_forward_noalloc(x: torch.Tensor, init_memories: torch.Tensor, n_heads: int,
                                dirs: int = 15, chunk: int = 0, out: torch.Tensor | None = None,
                                **kwargs) -> torch.Tensor:
    """hope_scan2d_forward through the entry point that allocates nothing: the route planes
    live in the library's own per-GPU device array (HOPE_NOALLOC_SCRATCH_BYTES), the batch
    runs in slices of whole images that fit it.  ``out`` must be given (this wrapper
    allocates nothing either); the other keyword arguments are those of hope_scan2d_forward
    except ``workspace``.  Calls that overlap in time on one GPU race on the scratch array."""
    if out is None:
        raise ValueError("out must be given: the no-allocation entry point allocates nothing")
    if kwargs.get("workspace") is not None:
        raise ValueError("the no-allocation entry point takes no workspace")
    kwargs.pop("workspace", None)
    return hope_scan2d_forward(x, init_memories, n_heads, dirs, chunk, out, _noalloc=True, **kwargs)


def hope_scan2d_backward_workspace_size(x: torch.Tensor, n_heads: int, dirs: int = 15,
                                        chunk: int = 0) -> int:
    lib = N.load_library()
    fm = make_fmap(x, n_heads)
    return int(lib.hope_scan2d_backward_workspace_size(ctypes.byref(fm), dirs, chunk, None))


def hope_scan2d_backward(x: torch.Tensor, init_memories: torch.Tensor, n_heads: int,
                         grad_out: torch.Tensor, dirs: int = 15, chunk: int = 0, *, stream=None,
                         eta_map: str = "sigmoid", eta_scale: float = 1.0, alpha_bias: float = 4.0,
                         eps: float = 1e-6, init_per_image: bool = False,
                         grad_x: torch.Tensor | None = None, grad_init: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, readout: str = "boundary"):
    """Gradients of sum(grad_out * hope_scan2d_forward(x, init_memories, ...)) with respect
    to x and init_memories; returns (grad_x, grad_init), float32, shaped like x and
    init_memories.  A workspace is allocated through torch when none is given.  readout
    "running" (the memory after the chunk's earlier tokens) is supported at d = 32."""
    lib = N.load_library()
    _require_device(x, "x")
    _require_device(init_memories, "init_memories")
    _require_device(grad_out, "grad_out")
    if init_memories.dtype != torch.float32 or not init_memories.is_contiguous():
        raise TypeError("init_memories must be a contiguous float32 tensor")
    if grad_out.dtype != torch.float32 or not grad_out.is_contiguous() or tuple(grad_out.shape) != tuple(x.shape):
        raise ValueError("grad_out must be a contiguous float32 tensor shaped like x")
    _check_numel(init_memories, state_numel(x, n_heads, init_per_image), "init_memories")
    if grad_x is None:
        grad_x = torch.empty(x.shape, dtype=torch.float32, device=x.device)
        _keep_for_stream(grad_x, stream)
    if grad_init is None:
        grad_init = torch.empty_like(init_memories)
        _keep_for_stream(grad_init, stream)
    for t, name in ((grad_x, "grad_x"), (grad_init, "grad_init")):
        _require_device(t, name)
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous float32 tensor")
    if tuple(grad_x.shape) != tuple(x.shape):
        raise ValueError("grad_x must be shaped like x")
    _check_numel(grad_init, init_memories.numel(), "grad_init")
    if workspace is None:
        nbytes = hope_scan2d_backward_workspace_size(x, n_heads, dirs, chunk)
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=x.device)
        _keep_for_stream(workspace, stream)
    fm = make_fmap(x, n_heads)
    opts = make_opts(stream, eta_map, eta_scale, alpha_bias, eps, init_per_image, None, workspace,
                     readout=readout)
    st = lib.hope_scan2d_backward(ctypes.byref(fm), init_memories.data_ptr(), dirs, chunk,
                                  grad_out.data_ptr(), grad_x.data_ptr(), grad_init.data_ptr(),
                                  ctypes.byref(opts))
    if st != N.HOPE_OK:
        raise HopeError(st, "hope_scan2d_backward")
    return grad_x, grad_init


def hope_debug_cross_scan(x: torch.Tensor, dirs: int = 15, routes: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """routes[slot, b, t, c] = x[b, p_r(t), c] for the selected routes (bit-exact)."""
    lib = N.load_library()
    _require_device(x, "x")
    B, H, W, D = x.shape
    n_sel = bin(dirs & 15).count("1")
    if routes is None:
        routes = torch.empty((max(n_sel, 1), B, H * W, D), dtype=x.dtype, device=x.device)
        _keep_for_stream(routes, stream)
    _require_device(routes, "routes")
    if routes.dtype != x.dtype:
        raise ValueError("routes must have the dtype of x")
    if routes.numel() < n_sel * B * H * W * D:
        raise ValueError(f"routes must hold {n_sel * B * H * W * D} elements")
    fm = make_fmap(x, 1)
    st = lib.hope_debug_cross_scan(ctypes.byref(fm), dirs, routes.data_ptr(), _stream_handle(stream))
    if st != N.HOPE_OK:
        raise HopeError(st, "hope_debug_cross_scan")
    return routes


def hope_debug_cross_merge(routes: torch.Tensor, H: int, W: int, dirs: int = 15,
                           out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """out[b, p, c] = sum over selected routes of routes[slot, b, p_r^-1(p), c] (fp32)."""
    lib = N.load_library()
    _require_device(routes, "routes")
    _, B, Nn, D = routes.shape
    if out is None:
        out = torch.empty((B, H, W, D), dtype=torch.float32, device=routes.device)
        _keep_for_stream(out, stream)
    _require_device(out, "out")
    if out.dtype != torch.float32:
        raise ValueError("out must be float32")
    if Nn != H * W or routes.shape[0] < bin(dirs & 15).count("1"):
        raise ValueError("routes must be [n_selected, B, H*W, D]")
    _check_numel(out, B * H * W * D, "out")
    st = lib.hope_debug_cross_merge(routes.data_ptr(), _dtype_code(routes), B, H, W, D, dirs,
                                    out.data_ptr(), _stream_handle(stream))
    if st != N.HOPE_OK:
        raise HopeError(st, "hope_debug_cross_merge")
    return out
