"""GPU parity of the VisionHOPE variants (Sec. 3.5 ablations, Eq. 26 direction scales,
App. B.5 skip) through the C ABI against the fp64 oracle, on the three scan kernels.

Counters of the step controls are integers decided by floating point: the GPU decides in
fp32, the oracle in fp64, and the quantities compared (eta and the two limits) come from
the projections of the fp32 state.  The counts must therefore agree exactly except on
tokens whose relative margin to the limit is within a band (counted by the oracle as
*_near).  The band is not the output tolerance: the state's products are split bf16
products (about 2^-16 relative), so the decision inputs are held far closer than a bf16
output is; COUNT_BAND is 2e-3 for a bf16 map (about a hundred times the split products'
error), the fp32 output tolerance for an fp32 map.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from _parity import TOL, check_final, check_out, to_device

pytestmark = pytest.mark.gpu

SHAPES = {
    "f32_d16": (2, 4, 6, 32, 2, "f32", 0),      # fp32 kernel
    "f32_d64": (1, 6, 9, 64, 1, "f32", 4),      # fp32 kernel, ragged chunks
    "bf16_d32": (2, 5, 37, 96, 3, "bf16", 0),   # chunk-parallel kernel, three token tiles
    "bf16_d64": (2, 6, 9, 128, 2, "bf16", 0),   # register-resident MFMA kernel, d = 64
    "bf16_d16": (2, 5, 20, 48, 3, "bf16", 0),   # chunk-parallel kernel, d = 16
    "bf16_d32_seg": (1, 3, 100, 32, 1, "bf16", 0),  # row chunks of 100: two segments of the chunk kernel
    "bf16_d64_seg": (1, 3, 40, 64, 1, "bf16", 0),   # d = 64, row chunks of 40: two segments
}
FROZEN = {"kv": ("k", "v"), "dynamics": ("eta", "alpha"), "q": ("q",)}
COUNT_BAND = {"f32": TOL["f32"], "bf16": 2e-3}

VARIANTS = {
    "scales_skip": dict(route_scales=True, skip=True),
    "hard_injection": dict(injection="hard"),
    "soft_spectral": dict(spectral="soft", eta_scale=3.0),
    "no_injection": dict(injection="none", eta_scale=0.05),
    "no_spectral": dict(spectral="none"),
    "frozen_kv": dict(frozen=("kv",)),
    "frozen_dynamics": dict(frozen=("dynamics",)),
    "frozen_all": dict(frozen=("kv", "dynamics", "q")),
    "no_dgd": dict(no_dgd=True),
    "shared_init": dict(shared_init=True),
    "counts": dict(counts=True, eta_scale=0.03),                     # eta near the injection limit
    "counts_spectral": dict(counts=True, eta_scale=4.0, alpha_bias=-2.0),  # low retention: spectral binds
    "queries": dict(queries=True),                                   # fixed outer query projection
}


def _run(shape, var, readout="boundary"):
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_forward
    B, H, W, D, nh, dt, chunk = shape
    d = D // nh
    inp = wl.draw(B, H, W, D, nh, seed=900 + H * 31 + W, dtype=dt, live=True)
    rng = np.random.Generator(np.random.PCG64(17))
    extra = {k: var[k] for k in ("eta_scale", "alpha_bias") if k in var}
    ok = dict(readout=readout, **extra)           # oracle keyword arguments
    gk = dict(readout=readout, **extra)           # GPU keyword arguments
    x, init = to_device(inp, dt)
    init_np = inp["init"]
    if var.get("route_scales"):
        lam = rng.uniform(0.5, 1.5, (4, D))
        ok["route_scales"] = lam
        gk["route_scales"] = torch.from_numpy(lam.astype(np.float32)).cuda()
    if var.get("skip"):
        sk = rng.standard_normal(D) * 0.3
        ok["skip"] = sk.astype(np.float32).astype(np.float64)
        gk["skip"] = torch.from_numpy(sk.astype(np.float32)).cuda()
    if "route_scales" in ok:
        ok["route_scales"] = ok["route_scales"].astype(np.float32).astype(np.float64)
    for k in ("injection", "spectral"):
        if k in var:
            ok[k] = gk[k] = var[k]
    if "frozen" in var:
        gk["frozen"] = var["frozen"]
        ok["frozen"] = tuple(m for f in var["frozen"] for m in FROZEN[f])
    if var.get("no_dgd"):
        gk["no_dgd"] = True
        ok["dgd"] = False
    if var.get("shared_init"):
        init_np = inp["init"][1]                       # [n_heads, S]
        init = torch.from_numpy(np.ascontiguousarray(init_np, dtype=np.float32)).cuda()
        ok["shared_init"] = gk["shared_init"] = True
    if var.get("queries"):
        q = rng.standard_normal((B, H, W, D)).astype(np.float32) * 0.7
        if dt == "bf16":
            qt = torch.from_numpy(q).to(torch.bfloat16)
            ok["queries"] = qt.float().numpy().astype(np.float64)
        else:
            qt = torch.from_numpy(q)
            ok["queries"] = q.astype(np.float64)
        gk["queries"] = qt.cuda()
    counts = None
    if var.get("counts"):
        counts = torch.zeros(3, dtype=torch.int64, device="cuda")
        gk["counts"] = counts
        ok["counts"] = {"near_rel": COUNT_BAND[dt]}
    fin = torch.full((B, 4, nh, 4 * d * d + 2 * d), float("nan"), dtype=torch.float32, device="cuda")
    out = hope_scan2d_forward(x, init, nh, 15, chunk, final_memories=fin, **gk)
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle.scan2d(inp["x"], init_np, nh, dirs=15, chunk=chunk, **ok)
    return out.cpu().numpy(), fin.cpu().numpy(), ref_out, ref_fin, d, (counts, ok.get("counts"))


@pytest.mark.parametrize("var", list(VARIANTS), ids=list(VARIANTS))
@pytest.mark.parametrize("shape", list(SHAPES), ids=list(SHAPES))
def test_variant_matches_oracle(shape, var):
    print("case", shape, var, flush=True)
    sh = SHAPES[shape]
    out, fin, ref_out, ref_fin, d, (cnt, ref_cnt) = _run(sh, VARIANTS[var])
    tol = TOL[sh[5]]
    e_out = check_out(out, ref_out, sh[4], tol)
    e_fin = check_final(fin, ref_fin, d, 15, tol)
    print(f"  rel_inf out {e_out:.2e} final {e_fin:.2e}", flush=True)
    if cnt is not None:
        got = cnt.cpu().numpy()
        assert got[0] == ref_cnt["updates"]
        assert abs(int(got[1]) - ref_cnt["inj"]) <= ref_cnt["inj_near"], (got, ref_cnt)
        assert abs(int(got[2]) - ref_cnt["spec"]) <= ref_cnt["spec_near"], (got, ref_cnt)
        if var == "counts":            # both outcomes of the injection test occur
            assert 0 < got[1] < got[0]
        else:                          # the spectral limit binds on some tokens
            assert got[2] > 0
        print(f"  counts {got.tolist()} oracle {ref_cnt} (differences "
              f"{int(got[1]) - ref_cnt['inj']}, {int(got[2]) - ref_cnt['spec']})", flush=True)


@pytest.mark.parametrize("shape", ["f32_d16", "bf16_d32", "bf16_d64"])
def test_variants_with_running_readout(shape):
    var = dict(route_scales=True, skip=True, frozen=("kv",), injection="hard", no_dgd=True,
               queries=True)
    print("case", shape, var, flush=True)
    sh = SHAPES[shape]
    out, fin, ref_out, ref_fin, d, _ = _run(sh, var, readout="running")
    tol = TOL[sh[5]]
    e_out = check_out(out, ref_out, sh[4], tol)
    e_fin = check_final(fin, ref_fin, d, 15, tol)
    print(f"  rel_inf out {e_out:.2e} final {e_fin:.2e}", flush=True)


# The two variant sets the benchmark times, at the full stage-3 size and launch
# configuration; the oracle checks sampled (image, head) slices (all four routes).
FULL_SETS = {
    "scales_skip_hard_injection": dict(route_scales=True, skip=True, injection="hard"),
    "frozen_kv_no_dgd_queries": dict(frozen=("kv",), no_dgd=True, queries=True),
}


@pytest.mark.parametrize("name", list(FULL_SETS), ids=list(FULL_SETS))
def test_variant_sets_full_size_stage3_sampled(name):
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_forward
    var = FULL_SETS[name]
    w = wl.WORKLOADS[3]
    images, heads = [0, 127], [0, 5]
    print(f"workload {w.name} variants {name}: images {images} heads {heads}", flush=True)
    inp = wl.draw_workload(w, live=True)
    x, init = to_device(inp, w.dtype)
    rng = np.random.Generator(np.random.PCG64(29))
    ok, gk = {}, {}
    if var.get("route_scales"):
        lam = rng.uniform(0.5, 1.5, (4, w.D)).astype(np.float32)
        ok["route_scales"] = lam.astype(np.float64)
        gk["route_scales"] = torch.from_numpy(lam).cuda()
    if var.get("skip"):
        sk = (rng.standard_normal(w.D) * 0.3).astype(np.float32)
        ok["skip"] = sk.astype(np.float64)
        gk["skip"] = torch.from_numpy(sk).cuda()
    if "injection" in var:
        ok["injection"] = gk["injection"] = var["injection"]
    if "frozen" in var:
        gk["frozen"] = var["frozen"]
        ok["frozen"] = tuple(m for f in var["frozen"] for m in FROZEN[f])
    if var.get("no_dgd"):
        gk["no_dgd"] = True
        ok["dgd"] = False
    if var.get("queries"):
        qt = torch.from_numpy(rng.standard_normal((w.B, w.H, w.W, w.D)).astype(np.float32) * 0.7).to(torch.bfloat16)
        ok["queries"] = qt.float().numpy().astype(np.float64)
        gk["queries"] = qt.cuda()
    d = w.d
    fin = torch.full((w.B, 4, w.n_heads, 4 * d * d + 2 * d), float("nan"), dtype=torch.float32, device="cuda")
    out = hope_scan2d_forward(x, init, w.n_heads, 15, w.chunk, final_memories=fin, **gk)
    torch.cuda.synchronize()
    ref_out, ref_fin = oracle.scan2d(inp["x"], inp["init"], w.n_heads, dirs=15, chunk=w.chunk,
                                     heads=heads, images=images, **ok)
    tol = TOL[w.dtype]
    e_out = check_out(out.cpu().numpy(), ref_out, w.n_heads, tol, heads=heads, images=images)
    e_fin = check_final(fin.cpu().numpy(), ref_fin, d, 15, tol, heads=heads, images=images)
    print(f"  rel_inf out {e_out:.2e} final {e_fin:.2e}", flush=True)


# The executed-step map (per token, at its pixel, by route and head) against the oracle's,
# on both kernels, with the default controls and with the controls binding on most tokens.
STEP_CASES = [
    ("f32_d16", {}),
    ("f32_d64", dict(eta_scale=50.0, alpha_bias=-3.0)),
    ("bf16_d32", {}),
    ("bf16_d64", {}),
    ("bf16_d64", dict(eta_scale=50.0, alpha_bias=-3.0)),
    ("bf16_d64", dict(injection="hard", route_scales=True)),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[f"{s}_{'_'.join(v) or 'default'}" for s, v in STEP_CASES])
def test_step_map_matches_oracle(case):
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_forward
    shape, var = case
    B, H, W, D, nh, dt, chunk = SHAPES[shape]
    print("case", shape, var, flush=True)
    d = D // nh
    inp = wl.draw(B, H, W, D, nh, seed=1300 + H * 31 + W, dtype=dt, live=True)
    x, init = to_device(inp, dt)
    extra = {k: var[k] for k in ("eta_scale", "alpha_bias", "injection") if k in var}
    gk, ok = dict(extra), dict(extra)
    if var.get("route_scales"):
        lam = np.random.Generator(np.random.PCG64(5)).uniform(0.5, 1.5, (4, D)).astype(np.float32)
        gk["route_scales"] = torch.from_numpy(lam).cuda()
        ok["route_scales"] = lam.astype(np.float64)
    sm = torch.full((B, 4, nh, H, W), float("nan"), dtype=torch.float32, device="cuda")
    out = hope_scan2d_forward(x, init, nh, 15, chunk, step_map=sm, **gk)
    torch.cuda.synchronize()
    ref_sm = np.full((B, 4, nh, H, W), np.nan)
    ref_out, _ = oracle.scan2d(inp["x"], inp["init"], nh, dirs=15, chunk=chunk, step_map=ref_sm, **ok)
    got = sm.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    e_step = float(np.max(np.abs(got - ref_sm)) / np.max(np.abs(ref_sm)))
    e_out = check_out(out.cpu().numpy(), ref_out, nh, TOL[dt])
    print(f"  rel_inf step {e_step:.2e} out {e_out:.2e}", flush=True)
    assert e_step <= TOL[dt]


def test_step_map_only_selected_routes():
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_forward
    B, H, W, D, nh, dt, chunk = SHAPES["bf16_d64"]
    inp = wl.draw(B, H, W, D, nh, seed=1400, dtype=dt, live=True)
    x, init = to_device(inp, dt)
    sm = torch.full((B, 4, nh, H, W), -7.0, dtype=torch.float32, device="cuda")
    hope_scan2d_forward(x, init, nh, 0b0110, chunk, step_map=sm)
    got = sm.cpu().numpy()
    assert np.all(got[:, [0, 3]] == -7.0)
    assert np.all(got[:, [1, 2]] > 0.0)


@pytest.mark.parametrize("shape,kw", [("bf16_d64", dict(readout="running")),
                                      ("bf16_d32", dict(readout="running")),
                                      ("f32_d64", dict(mem_chunk=2))],
                         ids=["bf16_d64_running", "bf16_d32_running", "f32_d64_mem_chunk2"])
def test_step_map_with_running_readout_and_two_chunk_sizes(shape, kw):
    import torch
    from self_modifying_memory_amd.scan2d import hope_scan2d_forward
    B, H, W, D, nh, dt, chunk = SHAPES[shape]
    print("case", shape, kw, flush=True)
    inp = wl.draw(B, H, W, D, nh, seed=1500 + H * 31 + W, dtype=dt, live=True)
    x, init = to_device(inp, dt)
    sm = torch.full((B, 4, nh, H, W), float("nan"), dtype=torch.float32, device="cuda")
    out = hope_scan2d_forward(x, init, nh, 15, chunk, step_map=sm, **kw)
    torch.cuda.synchronize()
    ref_sm = np.full((B, 4, nh, H, W), np.nan)
    ref_out, _ = oracle.scan2d(inp["x"], inp["init"], nh, dirs=15, chunk=chunk, step_map=ref_sm, **kw)
    got = sm.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    e_step = float(np.max(np.abs(got - ref_sm)) / np.max(np.abs(ref_sm)))
    e_out = check_out(out.cpu().numpy(), ref_out, nh, TOL[dt])
    print(f"  rel_inf step {e_step:.2e} out {e_out:.2e}", flush=True)
    assert e_step <= TOL[dt]
