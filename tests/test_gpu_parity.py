"""GPU parity of hope_scan2d_forward (through the C ABI) against the fp64 oracle.

Small cases run the oracle on the whole map; they span several token blocks,
ragged chunks, rectangles, every head dimension, route subsets and both gate
maps.  The full-size workloads run on the GPU at their real shape and launch
configuration and are compared on sampled (image, head) slices, which the oracle
computes exactly (all four routes of the slice).
"""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from _parity import TOL, check_final, check_out, run_gpu, to_device

pytestmark = pytest.mark.gpu

SMALL = [
    # B, H, W, D, nh, dtype, dirs, chunk, live, extra
    (1, 8, 8, 16, 1, "f32", 15, 0, False, {}),          # tiny workload as written: out == 0
    (1, 8, 8, 16, 1, "f32", 15, 0, True, {}),
    (2, 5, 7, 64, 2, "bf16", 15, 0, True, {}),          # rectangle, d = 32, two heads
    (1, 6, 9, 64, 1, "f32", 15, 4, True, {}),           # d = 64, chunk 4 does not divide 54
    (2, 3, 20, 48, 3, "f32", 15, 0, True, {}),          # d = 16, row chunks of 20 (> one block)
    (1, 17, 3, 32, 1, "bf16", 5, 0, True, {}),          # routes -> and down only
    (2, 4, 6, 32, 1, "f32", 2, 0, True, {}),            # a single route: no workspace
    (1, 4, 5, 32, 1, "f32", 15, 1, True, {}),           # chunk 1: token-wise recurrence
    (1, 4, 5, 32, 1, "f32", 15, 50, True, {}),          # one chunk longer than the map
    (1, 1, 13, 16, 1, "f32", 15, 0, True, {}),          # one row
    (1, 11, 1, 16, 1, "f32", 15, 0, True, {}),          # one column
    (2, 6, 6, 64, 2, "f32", 15, 0, True,
     dict(eta_map="softplus", eta_scale=0.025, alpha_bias=math.log(9.0))),  # VisionHOPE gates
    (1, 5, 5, 16, 1, "f32", 15, 0, True, dict(eta_scale=50.0, alpha_bias=-3.0)),  # clamps active
    (1, 40, 3, 32, 1, "f32", 12, 0, True, {}),          # column chunks of 40 tokens
    # bf16 maps with d = 32 / 64 run on the MFMA kernel
    (2, 6, 9, 128, 2, "bf16", 15, 0, True, {}),         # d = 64, row chunks 9, column chunks 6
    (1, 16, 16, 64, 1, "bf16", 15, 0, True, {}),        # d = 64, chunks of exactly 16
    (1, 20, 3, 64, 1, "bf16", 15, 0, True, {}),         # d = 64, column chunks 20 (> 16): chunk-parallel kernel
    (2, 5, 37, 96, 3, "bf16", 15, 0, True, {}),         # d = 32, row chunks 37: three token blocks
    (1, 9, 9, 32, 1, "bf16", 15, 33, True, {}),         # d = 32, chunk 33 over 81 tokens
    (2, 7, 7, 64, 2, "bf16", 8, 0, True, {}),           # d = 32, single route (no workspace)
    (1, 6, 6, 64, 1, "bf16", 15, 0, False, {}),         # d = 64 literal: out == 0
    (2, 5, 6, 64, 1, "bf16", 15, 0, True,
     dict(eta_map="softplus", eta_scale=0.025, alpha_bias=math.log(9.0))),
    (1, 5, 5, 32, 1, "bf16", 15, 0, True, dict(eta_scale=50.0, alpha_bias=-3.0)),  # clamps
    # d = 64 blocks staged during the gate phase: the next blocks start at the chunk ends
    (2, 6, 9, 64, 1, "bf16", 15, 5, True, {}),          # d = 64, chunk 5 over 54 tokens (ragged)
    (1, 4, 5, 64, 1, "bf16", 15, 1, True, {}),          # d = 64, one-token chunks
    (1, 5, 6, 64, 1, "bf16", 4, 7, True, {}),           # d = 64, one column route, chunk 7
    (1, 6, 6, 64, 1, "bf16", 15, 0, True, dict(eta_scale=50.0, alpha_bias=-3.0)),  # d = 64 clamps
]


def _case_id(c):
    B, H, W, D, nh, dt, dirs, chunk, live, extra = c
    return f"B{B}_{H}x{W}_D{D}h{nh}_{dt}_dirs{dirs}_c{chunk}_{'live' if live else 'lit'}" + \
        ("_" + "_".join(f"{k}{v:g}" if isinstance(v, float) else f"{k}{v}" for k, v in extra.items())
         if extra else "")


@pytest.mark.parametrize("case", SMALL, ids=[_case_id(c) for c in SMALL])
def test_small_maps_match_oracle(case):
    B, H, W, D, nh, dt, dirs, chunk, live, extra = case
    print("case", _case_id(case), flush=True)
    inp = wl.draw(B, H, W, D, nh, seed=B * 1000 + H * 37 + W, dtype=dt, live=live)
    out, fin = run_gpu(inp, nh, dt, dirs, chunk, **extra)
    ref_out, ref_fin = oracle.scan2d(inp["x"], inp["init"], nh, dirs=dirs, chunk=chunk, **extra)
    tol = TOL[dt]
    e_out = check_out(out, ref_out, nh, tol)
    e_fin = check_final(fin, ref_fin, D // nh, dirs, tol)
    if not live:
        assert np.all(out == 0.0)
    for r in range(4):                              # unselected routes leave final untouched
        if not (dirs >> r) & 1:
            assert np.all(np.isnan(fin[:, r]))
    print(f"  rel_inf out {e_out:.2e} final {e_fin:.2e}", flush=True)


def test_resume_from_final_state_on_gpu():
    # The final state of rows [0, k) resumes rows [k, H) of the row-major route.
    B, H, W, D = 2, 7, 5, 32
    inp = wl.draw(B, H, W, D, 1, seed=77, live=True)
    full, fin_full = run_gpu(inp, 1, "f32", dirs=1)
    k = 3
    a = {"x": np.ascontiguousarray(inp["x"][:, :k]), "init": inp["init"]}
    out_a, fin_a = run_gpu(a, 1, "f32", dirs=1)
    init_b = np.zeros((B, 4, 1, inp["init"].shape[-1]), dtype=np.float32)
    init_b[:, 0] = fin_a[:, 0]
    bpart = {"x": np.ascontiguousarray(inp["x"][:, k:]), "init": init_b}
    out_b, fin_b = run_gpu(bpart, 1, "f32", dirs=1, init_per_image=True)
    np.testing.assert_allclose(np.concatenate([out_a, out_b], 1), full, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(fin_b[:, 0], fin_full[:, 0], rtol=1e-5, atol=1e-6)


def test_deterministic_bitwise():
    w = wl.WORKLOADS[2].with_batch(8)
    inp = wl.draw_workload(w, live=True)
    o1, f1 = run_gpu(inp, w.n_heads, w.dtype)
    o2, f2 = run_gpu(inp, w.n_heads, w.dtype)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


@pytest.mark.parametrize("extra", [{}, dict(route_scales=True, skip=True)], ids=["default", "scales_skip"])
def test_stage3_image_independent_of_batch(extra):
    # the d = 64 kernel (gate-phase staging, shared Gram and retention tiles): an image's
    # outputs and final memories are bitwise the same alone and in a batch of six
    import torch
    w = wl.WORKLOADS[3].with_batch(6)
    inp = wl.draw_workload(w, live=True)
    one = dict(inp, x=inp["x"][:1], x_bits=inp["x_bits"][:1])
    kw = {}
    if extra:
        rng = np.random.Generator(np.random.PCG64(11))
        kw["route_scales"] = torch.from_numpy(rng.uniform(0.5, 1.5, (4, w.D)).astype(np.float32)).cuda()
        kw["skip"] = torch.from_numpy((rng.standard_normal(w.D) * 0.3).astype(np.float32)).cuda()
    o6, f6 = run_gpu(inp, w.n_heads, w.dtype, **kw)
    o1, f1 = run_gpu(one, w.n_heads, w.dtype, **kw)
    assert np.array_equal(o6[:1], o1) and np.array_equal(f6[:1], f1)


# Full-size workloads: the GPU runs the whole map; the oracle checks sampled slices.
SAMPLES = {1: ([0, 15], [0, 2]), 2: ([0, 63], [1, 5]), 3: ([0, 127], [0, 5]), 4: ([1], [2])}


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_full_size_workloads_sampled(idx):
    w = wl.WORKLOADS[idx]
    images, heads = SAMPLES[idx]
    print(f"workload {w.name}: images {images} heads {heads}", flush=True)
    inp = wl.draw_workload(w, live=True)
    out, fin = run_gpu(inp, w.n_heads, w.dtype)
    ref_out, ref_fin = oracle.scan2d(inp["x"], inp["init"], w.n_heads, heads=heads, images=images)
    e_out = check_out(out, ref_out, w.n_heads, TOL[w.dtype], heads=heads, images=images)
    e_fin = check_final(fin, ref_fin, w.d, 15, TOL[w.dtype], heads=heads, images=images)
    print(f"  rel_inf out {e_out:.2e} final {e_fin:.2e}", flush=True)


def test_full_size_literal_workload_reads_zero():
    # The workload as written (M_mem = 0) reads exactly zero everywhere (Eq. 46 fixed point).
    w = wl.WORKLOADS[3]
    inp = wl.draw_workload(w, live=False)
    out, fin = run_gpu(inp, w.n_heads, w.dtype)
    assert np.all(out == 0.0)
    assert np.all(fin[..., : w.d * w.d] == 0.0)
    ref_out, ref_fin = oracle.scan2d(inp["x"], inp["init"], w.n_heads, heads=[3], images=[64])
    check_final(fin, ref_fin, w.d, 15, TOL[w.dtype], heads=[3], images=[64])


BF16_OUT = [
    # B, H, W, D, nh, dtype, dirs, chunk
    (2, 5, 7, 64, 2, "bf16", 15, 0),    # MFMA kernel, four routes
    (1, 6, 9, 64, 1, "f32", 15, 4),     # fp32 kernel, ragged chunks
    (2, 7, 7, 64, 2, "bf16", 8, 0),     # one route: its own fp32 plane, then rounded
]


@pytest.mark.parametrize("case", BF16_OUT, ids=[f"B{c[0]}_{c[1]}x{c[2]}_D{c[3]}h{c[4]}_{c[5]}_dirs{c[6]}"
                                                  for c in BF16_OUT])
def test_bf16_out_is_the_fp32_sum_rounded_once(case):
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_forward

    B, H, W, D, nh, dt, dirs, chunk = case
    print("case", case, flush=True)
    inp = wl.draw(B, H, W, D, nh, seed=5000 + H * 37 + W, dtype=dt, live=True)
    x, init = to_device(inp, dt)
    o32 = hope_scan2d_forward(x, init, nh, dirs, chunk)
    o16 = hope_scan2d_forward(x, init, nh, dirs, chunk,
                              out=torch.empty(x.shape, dtype=torch.bfloat16, device=x.device))
    torch.cuda.synchronize()
    # the same fp32 sum, added in the same route order, rounded once to nearest even
    assert torch.equal(o16, o32.to(torch.bfloat16))
    ref, _ = oracle.scan2d(inp["x"], inp["init"], nh, dirs=dirs, chunk=chunk)
    e = check_out(o16.float().cpu().numpy(), ref, nh, TOL[dt] + 2.0 ** -8)
    print(f"  rel_inf out(bf16) {e:.2e}", flush=True)


def test_hires_long_memory_stress_sampled():
    # The high-resolution map with alpha-bias 8 (alpha ~ 0.9997): state carried across
    # 128 chunks of 128 tokens with almost no decay, checked on one (image, head) slice.
    w = wl.WORKLOADS[4]
    print(f"workload {w.name} alpha_bias 8: image 0 head 1", flush=True)
    inp = wl.draw_workload(w, live=True)
    out, fin = run_gpu(inp, w.n_heads, w.dtype, alpha_bias=8.0)
    ref_out, ref_fin = oracle.scan2d(inp["x"], inp["init"], w.n_heads, heads=[1], images=[0],
                                     alpha_bias=8.0)
    e_out = check_out(out, ref_out, w.n_heads, TOL[w.dtype], heads=[1], images=[0])
    e_fin = check_final(fin, ref_fin, w.d, 15, TOL[w.dtype], heads=[1], images=[0])
    print(f"  rel_inf out {e_out:.2e} final {e_fin:.2e}", flush=True)


# Running-state readout (y_t = M_mem,b G_{t-1} q_t) against the oracle's readout="running".
RUNNING = [
    # B, H, W, D, nh, dtype, dirs, chunk, extra
    (1, 8, 8, 16, 1, "f32", 15, 0, {}),            # fp32 kernel, d = 16
    (2, 3, 20, 48, 3, "f32", 15, 0, {}),           # fp32 kernel, row chunks of 20 (two blocks)
    (1, 6, 9, 64, 1, "f32", 15, 4, {}),            # fp32 kernel, d = 64, ragged chunks
    (2, 5, 7, 64, 2, "bf16", 15, 0, {}),           # MFMA d = 32, one block per chunk
    (2, 5, 37, 96, 3, "bf16", 15, 0, {}),          # MFMA d = 32, chunks of 37: three blocks
    (2, 6, 9, 128, 2, "bf16", 15, 0, {}),          # MFMA d = 64
    (1, 16, 16, 64, 1, "bf16", 15, 0, {}),         # MFMA d = 64, chunks of exactly 16
    (1, 20, 3, 64, 1, "bf16", 15, 0, {}),          # d = 64, column chunks of 20: running readout on the fp32 kernel
    (1, 5, 5, 32, 1, "bf16", 15, 0, dict(eta_scale=50.0, alpha_bias=-3.0)),  # clamps active
    (2, 5, 6, 64, 1, "bf16", 15, 0,
     dict(eta_map="softplus", eta_scale=0.025, alpha_bias=math.log(9.0))),
]


@pytest.mark.parametrize("case", RUNNING, ids=[_case_id(c[:8] + (True, c[8])) for c in RUNNING])
def test_running_readout_matches_oracle(case):
    B, H, W, D, nh, dt, dirs, chunk, extra = case
    print("case", case, flush=True)
    inp = wl.draw(B, H, W, D, nh, seed=7000 + B * 100 + H * 37 + W, dtype=dt, live=True)
    out, fin = run_gpu(inp, nh, dt, dirs, chunk, readout="running", **extra)
    ref_out, ref_fin = oracle.scan2d(inp["x"], inp["init"], nh, dirs=dirs, chunk=chunk,
                                     readout="running", **extra)
    e_out = check_out(out, ref_out, nh, TOL[dt])
    e_fin = check_final(fin, ref_fin, D // nh, dirs, TOL[dt])
    print(f"  rel_inf out {e_out:.2e} final {e_fin:.2e}", flush=True)


@pytest.mark.parametrize("shape", [(1, 5, 6, 32, 1, "f32"), (2, 5, 7, 64, 2, "bf16"),
                                   (1, 6, 6, 128, 2, "bf16")])
def test_running_readout_is_boundary_at_chunk_one(shape):
    # At one token per chunk the running memory is the chunk-start memory: bit for bit when
    # both readouts run on the same kernel, within the fp32 bar when the boundary readout
    # runs on the chunk-parallel kernel and the running one on the register-resident kernel
    from self_modifying_memory_amd.scan2d import hope_scan2d_kernel_name
    B, H, W, D, nh, dt = shape
    print("shape", shape, flush=True)
    inp = wl.draw(B, H, W, D, nh, seed=77, dtype=dt, live=True)
    x, _ = to_device(inp, dt)
    same = hope_scan2d_kernel_name(x, nh, 15, 1) == hope_scan2d_kernel_name(x, nh, 15, 1, readout="running")
    ob, fb = run_gpu(inp, nh, dt, 15, 1)
    orun, frun = run_gpu(inp, nh, dt, 15, 1, readout="running")
    if same:
        assert np.array_equal(ob, orun) and np.array_equal(fb, frun)
    else:
        e = float(np.max(np.abs(ob - orun)) / np.max(np.abs(orun)))
        ef = float(np.max(np.abs(fb - frun)) / np.max(np.abs(frun)))
        print(f"  boundary vs running: out {e:.2e} final {ef:.2e}", flush=True)
        assert e <= TOL["f32"] and ef <= TOL["f32"]


def test_running_readout_full_size_stage3_sampled():
    w = wl.WORKLOADS[3]
    images, heads = [0, 127], [0, 5]
    print(f"workload {w.name} running readout: images {images} heads {heads}", flush=True)
    inp = wl.draw_workload(w, live=True)
    out, fin = run_gpu(inp, w.n_heads, w.dtype, readout="running")
    ref_out, ref_fin = oracle.scan2d(inp["x"], inp["init"], w.n_heads, heads=heads, images=images,
                                     readout="running")
    e_out = check_out(out, ref_out, w.n_heads, TOL[w.dtype], heads=heads, images=images)
    e_fin = check_final(fin, ref_fin, w.d, 15, TOL[w.dtype], heads=heads, images=images)
    print(f"  rel_inf out {e_out:.2e} final {e_fin:.2e}", flush=True)
