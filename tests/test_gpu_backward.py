"""GPU parity of the backward pass (hope_scan2d_backward through the C ABI) against the
fp64 gradient oracle (oracle/hope_backward.py, autograd of the forward), on seeded maps
that span several chunks, ragged last chunks, both gate maps, per-image initial states,
route subsets and active step controls.

Metric: max |g - g_ref| / max |g_ref| over each gradient tensor (map, initial state),
held to the parity tolerance of the input dtype (1e-4 fp32, 2e-2 bf16; the backward
computes in fp32 throughout, on the map's values as given).  Rows of the initial state of
unselected routes must be exactly zero.
"""
import numpy as np
import pytest

import workloads as wl
from _parity import TOL, to_device
from oracle import hope_backward as hb

pytestmark = pytest.mark.gpu

#        B, H, W, D, nh, dtype, dirs, chunk, options
CASES = [
    (1, 4, 5, 32, 2, "f32", 15, 0, {}),                                   # d = 16, aligned chunks
    (1, 5, 6, 32, 1, "f32", 15, 4, dict(eta_scale=2.0)),                 # d = 32, ragged chunks
    (1, 4, 6, 64, 1, "f32", 15, 5, dict(eta_scale=2.0)),                 # d = 64
    (2, 3, 4, 64, 2, "bf16", 15, 0, {}),                                  # bf16 map, d = 32
    (1, 3, 5, 64, 1, "bf16", 15, 0, dict(eta_scale=2.0)),                # bf16 map, d = 64
    (1, 4, 4, 32, 1, "f32", 15, 3,
     dict(eta_map="softplus", eta_scale=0.5, alpha_bias=1.0)),           # softplus gates
    (1, 4, 4, 16, 1, "f32", 15, 2, dict(eta_scale=40.0, alpha_bias=-1.0)),  # clamps bind
    (2, 3, 4, 32, 1, "f32", 5, 0, dict(init_per_image=True)),             # routes 0 and 2, per image
    # d = 64 with chunks of at most 16 tokens (the chunk-parallel matrix-core kernel)
    (1, 3, 4, 64, 1, "f32", 15, 16, {}),                                  # one chunk, 12 of 16 slots
    (1, 4, 9, 64, 1, "f32", 15, 16, dict(eta_scale=2.0)),                # full 16-token chunks, tail 4
    (1, 4, 5, 64, 1, "f32", 15, 1, {}),                                   # one token per chunk
    (1, 4, 4, 64, 1, "f32", 15, 3,
     dict(eta_map="softplus", eta_scale=0.5, alpha_bias=1.0)),           # softplus gates
    (1, 4, 4, 64, 1, "f32", 15, 2, dict(eta_scale=40.0, alpha_bias=-1.0)),  # clamps bind
    (2, 3, 4, 128, 2, "f32", 5, 0, dict(init_per_image=True)),            # two heads, per image
    (1, 5, 7, 128, 2, "bf16", 10, 0, {}),                                 # routes 1 and 3, bf16
    (1, 3, 20, 64, 1, "f32", 15, 0, {}),                                  # d = 64, 20-token rows
    # the running readout (d = 32: the blocked kernel)
    (1, 5, 6, 32, 1, "f32", 15, 4, dict(eta_scale=2.0, readout="running")),   # ragged chunks
    (2, 3, 4, 64, 2, "bf16", 15, 0, dict(readout="running")),                  # bf16 map, two heads
]


def _id(c):
    B, H, W, D, nh, dt, dirs, chunk, kw = c
    tag = "_".join(f"{k}{v}" for k, v in kw.items())
    return f"B{B}_{H}x{W}_D{D}h{nh}_{dt}_dirs{dirs}_c{chunk}" + (f"_{tag}" if tag else "")


def _rel(got, ref):
    scale = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / scale) if scale > 0 else float(np.max(np.abs(got)))


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_backward_matches_gradient_oracle(case):
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_backward
    B, H, W, D, nh, dt, dirs, chunk, kw = case
    print("case", _id(case), flush=True)
    inp = wl.draw(B, H, W, D, nh, seed=9100 + H * 37 + W, dtype=dt, live=True)
    per_image = kw.get("init_per_image", False)
    init_np = inp["init"]
    if per_image:
        rng = np.random.Generator(np.random.PCG64(91))
        init_np = (init_np[None] * (1.0 + 0.1 * rng.standard_normal((B,) + init_np.shape))).astype(np.float32)
    g = np.random.Generator(np.random.PCG64(92)).standard_normal((B, H, W, D)).astype(np.float32)
    x, _ = to_device(inp, dt)
    init = torch.from_numpy(np.ascontiguousarray(init_np, dtype=np.float32)).cuda()
    gx, gi = hope_scan2d_backward(x, init, nh, torch.from_numpy(g).cuda(), dirs, chunk, **kw)
    torch.cuda.synchronize()
    gx, gi = gx.cpu().numpy(), gi.cpu().numpy()
    ref_x, ref_i = hb.scan2d_backward(inp["x"], init_np, nh, g, dirs=dirs, chunk=chunk, **kw)
    e_x, e_i = _rel(gx, ref_x), _rel(gi, ref_i)
    print(f"  rel grad_x {e_x:.2e} grad_init {e_i:.2e}", flush=True)
    assert e_x <= TOL[dt] and e_i <= TOL[dt]
    for r in range(4):                       # unselected routes: zero gradient rows
        if not (dirs >> r) & 1:
            assert np.all((gi[:, r] if per_image else gi[r]) == 0.0)


def test_backward_is_deterministic():
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_backward
    inp = wl.draw(2, 4, 5, 64, 2, seed=9200, dtype="bf16", live=True)
    x, init = to_device(inp, "bf16")
    g = torch.from_numpy(np.random.Generator(np.random.PCG64(93)).standard_normal((2, 4, 5, 64)).astype(np.float32)).cuda()
    a = [t.cpu().numpy() for t in hope_scan2d_backward(x, init, 2, g)]
    b = [t.cpu().numpy() for t in hope_scan2d_backward(x, init, 2, g)]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("idx", [3, 2])
def test_backward_full_size_content_memory_linear_response(idx):
    # The output is linear in the initial content memory M_mem (its trajectory is
    # M_mem,b G and G does not depend on it), so for any direction V of the M_mem rows
    #   <dL/dM_mem, V> = <grad_out, out(M_mem = V) - out(M_mem = 0)>
    # exactly; both sides come from the GPU (the backward, and two forward calls) at the
    # workload's full size and launch configuration.  The fp32 forward kernel is used on
    # both runs so that the two outputs share their arithmetic.
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_backward, hope_scan2d_forward
    w = wl.WORKLOADS[idx]
    print("workload", w.name, flush=True)
    inp = wl.draw_workload(w, live=True)
    x = torch.from_numpy(inp["x"].astype(np.float32)).cuda()      # the bf16 values, as fp32
    init_np = inp["init"].astype(np.float32)
    d = w.d
    rng = np.random.Generator(np.random.PCG64(94))
    g = torch.from_numpy(rng.standard_normal((w.B, w.H, w.W, w.D)).astype(np.float32)).cuda()
    V = rng.standard_normal((4, w.n_heads, d * d)).astype(np.float32) / np.sqrt(d)
    _, gi = hope_scan2d_backward(x, torch.from_numpy(init_np).cuda(), w.n_heads, g)
    lhs = float(np.sum(gi.cpu().numpy()[:, :, :d * d].astype(np.float64) * V))
    with_v, zero = init_np.copy(), init_np.copy()
    with_v[:, :, :d * d] = V
    zero[:, :, :d * d] = 0.0
    out_v = hope_scan2d_forward(x, torch.from_numpy(with_v).cuda(), w.n_heads)
    out_0 = hope_scan2d_forward(x, torch.from_numpy(zero).cuda(), w.n_heads)
    rhs = float(torch.sum((out_v.double() - out_0.double()) * g.double()).item())
    rel = abs(lhs - rhs) / max(abs(rhs), 1e-30)
    print(f"  <grad, V> {lhs:.6e}  linear response {rhs:.6e}  rel {rel:.2e}", flush=True)
    assert rel <= TOL["f32"]


def test_backward_full_size_stage3_image0():
    # The map gradient of one image depends only on that image's chains: the backward at
    # the full 128-image batch (the launch the benchmark times) against the gradient
    # oracle run on image 0 alone.  The backward computes in fp32 on the map's bf16 values,
    # held to the fp32 parity tolerance.
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_backward
    w = wl.WORKLOADS[3]
    print("workload", w.name, flush=True)
    inp = wl.draw_workload(w, live=True)
    x, init = to_device(inp, w.dtype)
    g = np.random.Generator(np.random.PCG64(95)).standard_normal((w.B, w.H, w.W, w.D)).astype(np.float32)
    gx, _ = hope_scan2d_backward(x, init, w.n_heads, torch.from_numpy(g).cuda())
    torch.cuda.synchronize()
    got = gx[0].cpu().numpy()
    ref, _ = hb.scan2d_backward(inp["x"][:1], inp["init"], w.n_heads, g[:1])
    e = _rel(got, ref[0])
    print(f"  rel grad_x[0] {e:.2e}", flush=True)
    assert e <= TOL["f32"]


#             B, H,   W,   D,  nh, dirs, options
LONG_CASES = [
    (1, 28, 28, 32, 1, 15, {}),                     # 28-token rows and columns (stage-2 chunks)
    (1, 6, 56, 32, 1, 3, {}),                       # 56-token rows (stage-1 chunks)
    (1, 56, 6, 32, 1, 12, dict(eta_scale=2.0)),     # 56-token columns
    (1, 4, 128, 32, 1, 3, {}),                      # 128-token rows (high-resolution chunks)
    (1, 128, 3, 32, 1, 12, dict(eta_scale=2.0)),    # 128-token columns
    (1, 2, 200, 32, 1, 3, {}),                      # 200-token rows: 13 blocks, the last of 8
    (2, 5, 12, 64, 2, 15, dict(chunk=20, init_per_image=True)),  # chunks of 20 (16 + 4) across rows
    (1, 6, 7, 32, 1, 15, dict(chunk=42, eta_map="softplus", eta_scale=0.5, alpha_bias=1.0)),  # one 42-token chunk
    (1, 4, 10, 32, 1, 15, dict(chunk=17, eta_scale=40.0, alpha_bias=-1.0)),  # 16 + 1 blocks, clamps bind
    # the running readout: the readout adjoint enters every earlier gain of the chunk
    (1, 28, 28, 32, 1, 15, dict(readout="running")),                        # stage-2 chunks
    (1, 4, 128, 32, 1, 3, dict(eta_scale=2.0, readout="running")),          # 128-token rows
    (2, 5, 12, 64, 2, 15, dict(chunk=20, init_per_image=True, readout="running")),
    (1, 6, 7, 32, 1, 15, dict(chunk=42, eta_map="softplus", eta_scale=0.5, alpha_bias=1.0,
                              readout="running")),
    (1, 4, 10, 32, 1, 15, dict(chunk=17, eta_scale=40.0, alpha_bias=-1.0, readout="running")),
]


def _long_id(c):
    tag = "_".join(f"{k}{v}" for k, v in c[6].items())
    return f"B{c[0]}_{c[1]}x{c[2]}_D{c[3]}_dirs{c[5]}" + (f"_{tag}" if tag else "")


@pytest.mark.parametrize("case", LONG_CASES, ids=[_long_id(c) for c in LONG_CASES])
def test_backward_long_chunks_match_gradient_oracle(case):
    # The chunk lengths of the stage-1, stage-2 and high-resolution workloads at d = 32:
    # several 16-token gate blocks and up to 128 gain rows per chunk, through the gain
    # adjoint (k, delta, the step, alpha) into grad_x and every memory's grad_init.  The
    # backward computes in fp32 on the bf16 map's values, so it is held to the fp32 bar.
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_backward
    B, H, W, D, nh, dirs, kw = case
    kw = dict(kw)
    chunk = kw.pop("chunk", 0)
    print("case", case, flush=True)
    inp = wl.draw(B, H, W, D, nh, seed=9300 + H + W, dtype="bf16", live=True,
                  init_per_image=kw.get("init_per_image", False))
    g = np.random.Generator(np.random.PCG64(96)).standard_normal((B, H, W, D)).astype(np.float32)
    x, init = to_device(inp, "bf16")
    gx, gi = hope_scan2d_backward(x, init, nh, torch.from_numpy(g).cuda(), dirs, chunk, **kw)
    torch.cuda.synchronize()
    ref_x, ref_i = hb.scan2d_backward(inp["x"], inp["init"], nh, g, dirs=dirs, chunk=chunk, **kw)
    e_x, e_i = _rel(gx.cpu().numpy(), ref_x), _rel(gi.cpu().numpy(), ref_i)
    print(f"  rel grad_x {e_x:.2e} grad_init {e_i:.2e}", flush=True)
    assert e_x <= TOL["f32"] and e_i <= TOL["f32"]


def test_backward_full_size_stage2_image0_head0():
    # The map gradient of one image's head slice depends only on that head's chains: the
    # backward at the full stage-2 batch (64 images, 6 heads of 32, 28-token chunks)
    # against the gradient oracle on image 0, head 0 alone.
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_backward
    w = wl.WORKLOADS[2]
    print("workload", w.name, flush=True)
    inp = wl.draw_workload(w, live=True)
    x, init = to_device(inp, w.dtype)
    g = np.random.Generator(np.random.PCG64(97)).standard_normal((w.B, w.H, w.W, w.D)).astype(np.float32)
    gx, _ = hope_scan2d_backward(x, init, w.n_heads, torch.from_numpy(g).cuda())
    torch.cuda.synchronize()
    d = w.d
    got = gx[0, ..., :d].cpu().numpy()
    ref, _ = hb.scan2d_backward(inp["x"][:1, ..., :d], inp["init"][:, :1], 1, g[:1, ..., :d])
    e = _rel(got, ref[0])
    print(f"  rel grad_x[0, head 0] {e:.2e}", flush=True)
    assert e <= TOL["f32"]


@pytest.mark.parametrize("D,nh,chunk", [(64, 2, 0), (64, 1, 0), (96, 3, 20)],
                         ids=["d32_aligned", "d64_aligned", "d32_chunk20"])
def test_backward_map_gradient_does_not_depend_on_batch(D, nh, chunk):
    # Every chain is one (image, head, route) and the route planes are summed per pixel in
    # a fixed order, so an image's map gradient is the same bit for bit whatever else is in
    # the batch (the initial-state gradient is a sum over the batch and is not compared).
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_backward
    B, H, W = 6, 5, 7
    inp = wl.draw(B, H, W, D, nh, seed=9400 + D + chunk, dtype="bf16", live=True)
    x, init = to_device(inp, "bf16")
    g = torch.from_numpy(np.random.Generator(np.random.PCG64(98)).standard_normal((B, H, W, D))
                         .astype(np.float32)).cuda()
    gx_all, _ = hope_scan2d_backward(x, init, nh, g, 15, chunk)
    gx_one, _ = hope_scan2d_backward(x[:1].contiguous(), init, nh, g[:1].contiguous(), 15, chunk)
    torch.cuda.synchronize()
    assert np.array_equal(gx_all[:1].cpu().numpy(), gx_one.cpu().numpy())
