"""GPU parity of the VisionHOPE block (hope_block_forward through the C ABI) against the
fp64 block oracle (oracle/hope_block.py), on seeded inputs and synthetic weights at
several head dimensions, a ragged chunk length, and image 0 of the full stage-3 batch.

Metric: max |(out - x) - (ref - x)| / max |ref - x|, the block's two branches measured
against their own scale (the residual x itself is passed through exactly).  The
projections take bf16 operands, so the bar is the bf16 parity tolerance, 2e-2.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import hope_block as hbk

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
_NAMES = {"init_memories": "init", "route_scales": "scales"}


def _device_weights(wts):
    import torch
    from self_modifying_memory_amd import _native as N
    dev = {}
    for name in N.BLOCK_WEIGHT_FIELDS:
        key = _NAMES.get(name, name)
        if key + "_bits" in wts:
            dev[name] = torch.from_numpy(wts[key + "_bits"].view(np.int16).copy()).view(torch.bfloat16).cuda()
        else:
            dev[name] = torch.from_numpy(np.ascontiguousarray(wts[key], dtype=np.float32)).cuda()
    return dev


def _oracle_weights(wts):
    return {k: v.astype(np.float64) for k, v in wts.items() if not k.endswith("_bits")}


def _rel_branch(got, ref, x):
    d_ref = ref - x
    return float(np.max(np.abs((got - x) - d_ref)) / np.max(np.abs(d_ref)))


#        B, H, W, D, D_m, nh, ffn, chunk
CASES = [
    (1, 4, 5, 128, 128, 2, 512, 0),     # d = 64
    (2, 3, 7, 128, 128, 4, 256, 3),     # d = 32, ragged chunks
    (1, 5, 4, 128, 128, 8, 512, 0),     # d = 16
    (1, 6, 6, 256, 256, 4, 1024, 0),    # d = 64, wider
    (3, 9, 10, 128, 128, 2, 256, 5),    # d = 64, 270 pixels: three GEMM row tiles, the last ragged
    (1, 4, 6, 512, 512, 8, 512, 0),     # d = 64, D = 512: eight values per lane in the LayerNorm
    # the pages' evaluated form (VisionHOPE App. C.3): D_m = D / 2, n_heads = D / 32 heads of 16
    (1, 14, 14, 384, 192, 12, 1536, 0),  # stage-3 width: ragged GEMM N (192) and K (192)
    (2, 9, 8, 192, 96, 6, 768, 0),       # stage-2 width: D % 128 != 0 (CPE and LayerNorm apart)
    (1, 8, 8, 96, 48, 3, 384, 0),        # stage-1 width: K = 48 (a half MFMA k-step)
    (1, 6, 7, 96, 48, 3, 400, 5),        # ffn_dim not a multiple of 32, ragged chunks
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_{c[1]}x{c[2]}_D{c[3]}m{c[4]}h{c[5]}_F{c[6]}_c{c[7]}" for c in CASES])
def test_block_matches_oracle(case):
    import torch
    from self_modifying_memory_amd.block import hope_block_forward
    B, H, W, D, Dm, nh, F, chunk = case
    print("case", case, flush=True)
    x = np.random.Generator(np.random.PCG64(500 + D + H)).standard_normal((B, H, W, D)).astype(np.float32)
    wts = wl.draw_block_weights(D, nh, F, seed=600 + D + W, D_m=Dm)
    out = hope_block_forward(torch.from_numpy(x).cuda(), _device_weights(wts), nh, F, chunk, D_m=Dm)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = hbk.block_forward(x, _oracle_weights(wts), nh, chunk=chunk)
    e = _rel_branch(got, ref, x.astype(np.float64))
    print(f"  rel branch error {e:.2e}", flush=True)
    assert e <= TOL_BF16


def test_block_is_deterministic():
    import torch
    from self_modifying_memory_amd.block import hope_block_forward
    x = torch.from_numpy(np.random.Generator(np.random.PCG64(7)).standard_normal((2, 5, 6, 128)).astype(np.float32)).cuda()
    w = _device_weights(wl.draw_block_weights(128, 4, 512, seed=8, D_m=64))
    a = hope_block_forward(x, w, 4, D_m=64).cpu().numpy()
    b = hope_block_forward(x, w, 4, D_m=64).cpu().numpy()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("Dm_half", [False, True], ids=["Dm=D_6x64", "Dm=D/2_12x16"])
def test_block_full_size_stage3_image0(Dm_half):
    # every step of the block is per image, so image 0 of the full 128-image batch (the
    # launch the benchmark times) is checked against the oracle run on image 0 alone; once
    # at D_m = D with the scan workload's heads, once in the pages' evaluated form
    import torch
    from self_modifying_memory_amd.block import hope_block_forward
    w = wl.WORKLOADS[3]
    Dm, nh = (w.D // 2, w.D // 32) if Dm_half else (w.D, w.n_heads)
    print("workload", w.name, "D_m", Dm, "heads", nh, flush=True)
    F = 4 * w.D
    x = np.random.Generator(np.random.PCG64(31)).standard_normal((w.B, w.H, w.W, w.D)).astype(np.float32)
    wts = wl.draw_block_weights(w.D, nh, F, seed=32, D_m=Dm)
    out = hope_block_forward(torch.from_numpy(x).cuda(), _device_weights(wts), nh, F, D_m=Dm)
    torch.cuda.synchronize()
    got = out[0:1].cpu().numpy().astype(np.float64)
    ref = hbk.block_forward(x[:1], _oracle_weights(wts), nh)
    e = _rel_branch(got, ref, x[:1].astype(np.float64))
    print(f"  rel branch error image 0 {e:.2e}", flush=True)
    assert e <= TOL_BF16
