"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the fp64 oracle by the normwise metric.

Metric: rel_inf = max|o - o_ref| / max|o_ref| per (image, head) slice of the
output, and per row and per column of that slice (the aligned chunks of the row and
column routes, so that late tokens are held to the same relative bar), and per (image,
route, head, memory) block of the final state.  A block
whose reference is identically zero must be exactly zero; a block whose reference
is below 1e-30 (fp32 state in the denormal range) is held to an absolute bound
of 1e-30 * tol instead.
Tolerances: fp32 inputs 1e-4, bf16 inputs 2e-2.
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}
MEM_NAMES = ("mem", "k", "v", "q", "eta", "alpha")


def to_device(inp: dict, dtype: str):
    import torch
    if dtype == "bf16":
        x = torch.from_numpy(inp["x_bits"].view(np.int16).copy()).view(torch.bfloat16)
    else:
        x = torch.from_numpy(np.ascontiguousarray(inp["x"], dtype=np.float32))
    init = torch.from_numpy(np.ascontiguousarray(inp["init"], dtype=np.float32))
    return x.cuda(), init.cuda()


def run_gpu(inp: dict, n_heads: int, dtype: str, dirs: int = 15, chunk: int = 0, final: bool = True,
            **kw):
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_forward
    x, init = to_device(inp, dtype)
    B = x.shape[0]
    d = x.shape[3] // n_heads
    fin = None
    if final:
        fin = torch.full((B, 4, n_heads, 4 * d * d + 2 * d), float("nan"), dtype=torch.float32,
                         device=x.device)
    out = hope_scan2d_forward(x, init, n_heads, dirs, chunk, final_memories=fin, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (fin.cpu().numpy() if fin is not None else None)


def rel_inf(got: np.ndarray, ref: np.ndarray, tol: float) -> float:
    """Normwise error of one block (see module docstring); returns the ratio to tol."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(got)):
        return np.inf
    m = np.abs(ref).max() if ref.size else 0.0
    diff = np.abs(got - ref).max() if ref.size else 0.0
    if m == 0.0:
        return 0.0 if diff == 0.0 else np.inf
    if m < 1e-30:
        return diff / (1e-30 * tol) * tol
    return diff / m


def check_out(got, ref, n_heads: int, tol: float, heads=None, images=None) -> float:
    """Per (image, head) rel_inf of out; returns the worst, asserts <= tol."""
    B = ref.shape[0]
    d = ref.shape[-1] // len(heads if heads is not None else range(n_heads))
    heads = list(range(n_heads)) if heads is None else list(heads)
    images = list(range(B)) if images is None else list(images)
    worst = 0.0
    for bi, b in enumerate(images):
        for hi, h in enumerate(heads):
            g_bh = got[b, ..., h * d:(h + 1) * d]
            r_bh = ref[bi, ..., hi * d:(hi + 1) * d]
            e = rel_inf(g_bh, r_bh, tol)
            assert e <= tol, f"out image {b} head {h}: rel_inf {e:.3e} > {tol}"
            worst = max(worst, e)
            # per chunk as well (rows are the row routes' aligned chunks, columns the column
            # routes'), so that late tokens with small outputs are held to the same relative
            # bar; a chunk whose reference lies below 1e-30 takes the absolute bound
            if g_bh.ndim == 3:
                for y in range(r_bh.shape[0]):
                    e = rel_inf(g_bh[y], r_bh[y], tol)
                    assert e <= tol, f"out image {b} head {h} row {y}: rel_inf {e:.3e} > {tol}"
                for x in range(r_bh.shape[1]):
                    e = rel_inf(g_bh[:, x], r_bh[:, x], tol)
                    assert e <= tol, f"out image {b} head {h} column {x}: rel_inf {e:.3e} > {tol}"
    return worst


def check_final(got, ref, d: int, dirs: int, tol: float, heads=None, images=None) -> float:
    """Per (image, route, head, memory) rel_inf of the final state."""
    dd = d * d
    spans = [(i * dd, (i + 1) * dd) for i in range(4)] + [(4 * dd, 4 * dd + d), (4 * dd + d, 4 * dd + 2 * d)]
    nh_ref = ref.shape[2]
    heads = list(range(nh_ref)) if heads is None else list(heads)
    images = list(range(ref.shape[0])) if images is None else list(images)
    worst = 0.0
    for bi, b in enumerate(images):
        for r in range(4):
            if not (dirs >> r) & 1:
                continue
            for hi, h in enumerate(heads):
                for name, (lo, hi_) in zip(MEM_NAMES, spans):
                    e = rel_inf(got[b, r, h, lo:hi_], ref[bi, r, hi, lo:hi_], tol)
                    assert e <= tol, f"final image {b} route {r} head {h} {name}: {e:.3e} > {tol}"
                    worst = max(worst, e)
    return worst
