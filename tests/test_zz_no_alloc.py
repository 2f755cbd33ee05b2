"""The entry point that allocates nothing (hope_scan2d_forward_noalloc, through the C ABI)
against the allocating forward (hope_scan2d_forward) on the same inputs: two calls in a
row, the second on a smaller input, each compared element by element (the two run the
same kernels on the same chains, so the results must be identical bit for bit).  The
first call needs two slices of images to fit the route planes in the library's scratch
array; one case also moves every per-image pointer (per-image initial state, final state,
step map) across the slices."""
import numpy as np
import pytest

import workloads as wl
from _parity import to_device

pytestmark = pytest.mark.gpu


def _both(x, init, nh, chunk=0, out_dtype=None, **kw):
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_forward, hope_scan2d_forward_noalloc
    dt = torch.float32 if out_dtype is None else out_dtype
    ref = hope_scan2d_forward(x, init, nh, 15, chunk, torch.empty(x.shape, dtype=dt, device=x.device), **kw)
    got = hope_scan2d_forward_noalloc(x, init, nh, 15, chunk,
                                      torch.full(x.shape, float("nan"), dtype=dt, device=x.device), **kw)
    torch.cuda.synchronize()
    return ref.cpu(), got.cpu()


def test_noalloc_matches_forward_twice_second_smaller():
    import torch
    from self_modifying_memory_amd import _native as N
    w = wl.WORKLOADS[3]
    print("first call:", w.name, flush=True)
    inp = wl.draw_workload(w, live=True)
    x, init = to_device(inp, w.dtype)
    assert 3 * w.B * w.H * w.W * w.D * 4 > N.HOPE_NOALLOC_SCRATCH_BYTES  # two slices
    ref, got = _both(x, init, w.n_heads)
    assert torch.equal(ref, got)
    print("second call: B3 6x7 D64 nh2 chunk 5", flush=True)
    small = wl.draw(3, 6, 7, 64, 2, seed=77, dtype="bf16", live=True)
    xs, inits = to_device(small, "bf16")
    ref, got = _both(xs, inits, 2, chunk=5)
    assert torch.equal(ref, got)


def test_noalloc_per_image_pointers_across_slices():
    import torch
    from self_modifying_memory_amd import _native as N
    B, H, W, D, nh = 40, 28, 28, 192, 6
    per_image = 3 * H * W * D * 4
    assert per_image * B > N.HOPE_NOALLOC_SCRATCH_BYTES > per_image  # several slices
    print("call: B40 28x28 D192 nh6, per-image init, final state, step map, counts", flush=True)
    inp = wl.draw(B, H, W, D, nh, seed=78, dtype="bf16", live=True, init_per_image=True)
    x, init = to_device(inp, "bf16")
    S = 4 * 32 * 32 + 2 * 32
    outs = []
    for _ in range(2):
        fin = torch.full((B, 4, nh, S), float("nan"), device=x.device)
        steps = torch.full((B, 4, nh, H, W), float("nan"), device=x.device)
        cnt = torch.zeros(3, dtype=torch.int64, device=x.device)
        outs.append(dict(final_memories=fin, step_map=steps, counts=cnt))
    import torch as _t
    from self_modifying_memory_amd.scan2d import hope_scan2d_forward, hope_scan2d_forward_noalloc
    ref = hope_scan2d_forward(x, init, nh, 15, 0, _t.empty(x.shape, device=x.device), init_per_image=True,
                              **outs[0])
    got = hope_scan2d_forward_noalloc(x, init, nh, 15, 0, _t.full(x.shape, float("nan"), device=x.device),
                                      init_per_image=True, **outs[1])
    _t.cuda.synchronize()
    assert _t.equal(ref.cpu(), got.cpu())
    for k in ("final_memories", "step_map", "counts"):
        assert _t.equal(outs[0][k].cpu(), outs[1][k].cpu()), k
    print("second call: B2 5x9 D64 nh1, bf16 out", flush=True)
    small = wl.draw(2, 5, 9, 64, 1, seed=79, dtype="bf16", live=True)
    xs, inits = to_device(small, "bf16")
    ref, got = _both(xs, inits, 1, out_dtype=_t.bfloat16)
    assert _t.equal(ref.view(_t.int16), got.view(_t.int16))
