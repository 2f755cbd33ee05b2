"""GPU: the route permutations alone, bit-exact against the oracle's orders.

Orders: "VMamba: Visual State Space Model" (explainer), the printed four orders on a
3x4 grid and the restore-then-sum merge; "VisionHOPE: Visual Backbones as
Self-Modifying Learning Systems" Sec. 2.3 Eq. 24 and Eq. 26.
"""
import os

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU test needs a visible GPU"
    return torch


@pytest.mark.parametrize("H,W,D", [(3, 4, 16), (5, 7, 24), (1, 9, 8), (8, 1, 4), (16, 16, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cross_scan_bit_exact(H, W, D, dtype):
    torch = _torch()
    from self_modifying_memory_amd.scan2d import hope_debug_cross_scan
    print(f"cross_scan H={H} W={W} D={D} {dtype}", flush=True)
    inp = wl.draw(2, H, W, D, 1, seed=H * 100 + W, dtype=dtype)
    if dtype == "bf16":
        bits = inp["x_bits"]
        x = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    else:
        bits = inp["x"].view(np.uint32)
        x = torch.from_numpy(inp["x"].copy()).cuda()
    for dirs in range(1, 16):
        routes = hope_debug_cross_scan(x, dirs)
        torch.cuda.synchronize()
        got = routes.cpu().view(torch.int16 if dtype == "bf16" else torch.int32).numpy()
        slots = [r for r in range(4) if (dirs >> r) & 1]
        for s, r in enumerate(slots):
            want = bits.reshape(2, H * W, D)[:, oracle.route_order(H, W, r), :]
            assert np.array_equal(got[s].view(want.dtype), want), (dirs, r)


def test_cross_scan_reproduces_printed_3x4_orders():
    torch = _torch()
    from self_modifying_memory_amd.scan2d import hope_debug_cross_scan
    x = torch.arange(12, dtype=torch.float32).reshape(1, 3, 4, 1).cuda()
    routes = hope_debug_cross_scan(x, 15).cpu().numpy()
    by_name = {"row_fwd": 0, "row_rev": 1, "col_fwd": 2, "col_rev": 3}
    with open(os.path.join(GOLDEN, "cross_scan_3x4.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, *vals = line.split()
            assert routes[by_name[name], 0, :, 0].astype(int).tolist() == [int(v) for v in vals]


@pytest.mark.parametrize("H,W", [(3, 4), (6, 5), (1, 7)])
def test_cross_merge_matches_oracle_and_identity(H, W):
    torch = _torch()
    from self_modifying_memory_amd.scan2d import hope_debug_cross_merge, hope_debug_cross_scan
    rng = np.random.Generator(np.random.PCG64(7))
    B, D = 2, 12
    ys = rng.standard_normal((4, B, H * W, D)).astype(np.float32)
    for dirs in (15, 1, 6, 9):
        slots = [r for r in range(4) if (dirs >> r) & 1]
        routes = torch.from_numpy(ys[: len(slots)].copy()).cuda()
        out = hope_debug_cross_merge(routes, H, W, dirs).cpu().numpy()
        want = oracle.cross_merge({r: ys[s].astype(np.float64) for s, r in enumerate(slots)}, H, W)
        np.testing.assert_allclose(out, want, rtol=1e-6, atol=1e-6)
    # identity scans: merge(scan(x)) is exactly 4x for bf16-valued x
    xv, xb = wl.round_to_bf16(rng.standard_normal((B, H, W, D)).astype(np.float32))
    for dt in ("f32", "bf16"):
        if dt == "bf16":
            x = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).cuda()
        else:
            x = torch.from_numpy(xv.copy()).cuda()
        out = hope_debug_cross_merge(hope_debug_cross_scan(x, 15), H, W, 15).cpu().numpy()
        assert np.array_equal(out, 4.0 * xv)
