"""GPU parity of the chunk-parallel kernel (chain_chunk_kernel: bf16 maps, d = 16, 32, 64,
boundary readout) against the fp64 oracle, through the C ABI: token-tile counts from one to
a full segment, ragged tiles and chunks, chunks that span several segments (the gain carried
between segments), one-token chunks, active step controls and the VisionHOPE gate maps.
Every case first asserts which kernel the call runs on."""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from _parity import TOL, check_final, check_out, run_gpu, to_device

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, W, D, nh, dirs, chunk, extra
    (1, 8, 8, 16, 1, 15, 0, {}),            # d = 16, one tile of 8 tokens
    (2, 14, 14, 48, 3, 15, 0, {}),          # d = 16, chunks of 14 (the stage-3 block shape)
    (1, 6, 40, 16, 1, 15, 0, {}),           # d = 16, row chunks of 40: three tiles, the last ragged
    (1, 3, 128, 32, 2, 3, 0, {}),           # d = 16, row chunks of 128: one full segment
    (1, 2, 150, 16, 1, 3, 0, {}),           # d = 16, row chunks of 150: two segments
    (1, 5, 9, 16, 1, 15, 17, {}),           # d = 16, chunk 17 over 45 tokens (ragged)
    (1, 4, 6, 16, 1, 15, 1, {}),            # d = 16, one token per chunk
    (2, 5, 37, 64, 2, 15, 0, {}),           # d = 32, row chunks of 37
    (1, 4, 64, 32, 1, 3, 0, {}),            # d = 32, chunks of exactly one segment
    (1, 3, 65, 32, 1, 3, 0, {}),            # d = 32, a segment of 64 and one of 1
    (1, 2, 128, 32, 1, 3, 0, {}),           # d = 32, two full segments
    (1, 2, 200, 32, 1, 3, 0, {}),           # d = 32, four segments, the last of 8
    (1, 9, 9, 32, 1, 15, 33, {}),           # d = 32, chunk 33 over 81 tokens
    (1, 4, 5, 32, 1, 15, 1, {}),            # d = 32, one token per chunk
    (1, 40, 3, 32, 1, 12, 0, {}),           # d = 32, column chunks of 40
    (1, 5, 70, 32, 1, 15, 0, dict(eta_scale=50.0, alpha_bias=-3.0)),  # clamps bind, two segments
    (1, 6, 20, 32, 1, 15, 0, dict(eta_scale=50.0, alpha_bias=-3.0)),  # d = 16 x 2 heads, clamps
    (2, 6, 30, 64, 2, 15, 0,
     dict(eta_map="softplus", eta_scale=0.025, alpha_bias=math.log(9.0))),  # VisionHOPE gates
    (1, 4, 140, 16, 1, 3, 0, dict(alpha_bias=8.0)),  # long memory, two d = 16 segments
    (1, 3, 20, 64, 1, 15, 0, {}),           # d = 64, row chunks of 20: one segment of two tiles
    (1, 2, 40, 64, 1, 3, 0, {}),            # d = 64, row chunks of 40: segments of 32 and 8
    (2, 5, 33, 128, 2, 15, 0, {}),          # d = 64, two heads, a segment of 32 and one of 1
    (1, 6, 9, 64, 1, 15, 17, {}),           # d = 64, chunk 17 over 54 tokens
    (1, 4, 28, 64, 1, 15, 0, dict(eta_scale=50.0, alpha_bias=-3.0)),  # d = 64, clamps bind
]


def _id(c):
    B, H, W, D, nh, dirs, chunk, extra = c
    tag = "_".join(f"{k}{v:g}" if isinstance(v, float) else f"{k}{v}" for k, v in extra.items())
    return f"B{B}_{H}x{W}_D{D}h{nh}_dirs{dirs}_c{chunk}" + (f"_{tag}" if tag else "")


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_chunk_kernel_matches_oracle(case):
    from self_modifying_memory_amd.scan2d import hope_scan2d_kernel_name
    B, H, W, D, nh, dirs, chunk, extra = case
    print("case", _id(case), flush=True)
    inp = wl.draw(B, H, W, D, nh, seed=6100 + B * 100 + H * 37 + W, dtype="bf16", live=True)
    x, _ = to_device(inp, "bf16")
    # d = 16 always runs on this kernel; d = 32 and d = 64 when some chunk is longer than 16
    # tokens (shorter ones go to the register-resident kernel, checked here as well)
    d = D // nh
    routes = [r for r in range(4) if (dirs >> r) & 1]
    longest = max(min(chunk or (W if r < 2 else H), H * W) for r in routes)
    on_chunk = d == 16 or (d == 32 and longest > 16) or (d == 64 and longest > 16)
    want = "chain_chunk_kernel" if on_chunk else "chain_mfma_kernel"
    assert hope_scan2d_kernel_name(x, nh, dirs, chunk) == want
    out, fin = run_gpu(inp, nh, "bf16", dirs, chunk, **extra)
    ref_out, ref_fin = oracle.scan2d(inp["x"], inp["init"], nh, dirs=dirs, chunk=chunk, **extra)
    e_out = check_out(out, ref_out, nh, TOL["bf16"])
    e_fin = check_final(fin, ref_fin, D // nh, dirs, TOL["bf16"])
    for r in range(4):
        if not (dirs >> r) & 1:
            assert np.all(np.isnan(fin[:, r]))
    print(f"  rel_inf out {e_out:.2e} final {e_fin:.2e}", flush=True)


def test_chunk_kernel_literal_reads_zero():
    # M_mem = 0 stays 0 under the shared gain (Eq. 46): the literal workload reads zero exactly
    inp = wl.draw(2, 6, 70, 64, 2, seed=6200, dtype="bf16", live=False)
    out, fin = run_gpu(inp, 2, "bf16", 15, 0)
    assert np.all(out == 0.0)
    assert np.all(fin[..., : 32 * 32] == 0.0)


def test_chunk_kernel_is_deterministic():
    inp = wl.draw(4, 12, 70, 96, 3, seed=6300, dtype="bf16", live=True)
    o1, f1 = run_gpu(inp, 3, "bf16")
    o2, f2 = run_gpu(inp, 3, "bf16")
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


@pytest.mark.parametrize("shape", [(10, 28), (4, 56), (3, 128)], ids=["rows28", "rows56", "rows128"])
def test_chunk_kernel_result_does_not_depend_on_batch_size(shape):
    # at d = 32 a call with at most 256 chains runs 16 waves per chain (two per state-row tile,
    # their carry shares added at the chunk end), a larger one 8; the 8-wave form keeps the
    # same two shares, so an image's result is bitwise the same in a batch of 2 and of 72
    H, W = shape
    big = wl.draw(72, H, W, 32, 1, seed=6400 + W, dtype="bf16", live=True)
    small = {k: (v[:2] if k in ("x", "x_bits") else v) for k, v in big.items()}
    print("shape", shape, flush=True)
    o_big, f_big = run_gpu(big, 1, "bf16")
    o_small, f_small = run_gpu(small, 1, "bf16")
    assert np.array_equal(o_big[:2], o_small) and np.array_equal(f_big[:2], f_small)
