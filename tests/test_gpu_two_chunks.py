"""GPU parity of the two chunk sizes of "Nested Learning" (one for the working memory,
one for the projection memories) through the C ABI against the fp64 oracle.

The working memory M_mem keeps its boundary state (boundary readout and self-generated
targets) over chunks of mem_chunk tokens, the other five memories over the projection
chunk; the library runs these calls on the fp32 chain kernel for every dtype.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from _parity import TOL, check_final, check_out, run_gpu

pytestmark = pytest.mark.gpu

#        B, H, W, D, nh, dtype, chunk, mem_chunk, readout
CASES = [
    (2, 5, 7, 32, 2, "f32", 0, 3, "boundary"),      # aligned projection chunks 7 / 5, memory 3
    (1, 6, 9, 32, 1, "f32", 4, 6, "boundary"),      # grids 4 and 6 interleave
    (1, 6, 9, 32, 1, "f32", 4, 6, "running"),       # running readout on the memory's own gain
    (1, 4, 6, 64, 1, "f32", 5, 2, "boundary"),      # d = 64, memory chunk shorter
    (2, 5, 37, 96, 3, "bf16", 0, 16, "boundary"),   # bf16 map, d = 32
    (1, 6, 9, 64, 1, "bf16", 4, 3, "boundary"),     # bf16 map, d = 64
    (1, 5, 5, 32, 1, "f32", 3, 100, "boundary"),    # memory chunk longer than the sequence
    (1, 5, 6, 16, 1, "f32", 4, 4, "boundary"),      # equal lengths: the one-size operator
]


def _id(c):
    B, H, W, D, nh, dt, chunk, cm, ro = c
    return f"B{B}_{H}x{W}_D{D}h{nh}_{dt}_c{chunk}_m{cm}_{ro}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_two_chunk_sizes_match_oracle(case):
    B, H, W, D, nh, dt, chunk, cm, ro = case
    print("case", _id(case), flush=True)
    inp = wl.draw(B, H, W, D, nh, seed=8100 + H * 37 + W, dtype=dt, live=True)
    out, fin = run_gpu(inp, nh, dt, 15, chunk, mem_chunk=cm, readout=ro, eta_scale=2.0)
    ref_out, ref_fin = oracle.scan2d(inp["x"], inp["init"], nh, dirs=15, chunk=chunk, mem_chunk=cm,
                                     readout=ro, eta_scale=2.0)
    tol = TOL[dt]
    e_out = check_out(out, ref_out, nh, tol)
    e_fin = check_final(fin, ref_fin, D // nh, 15, tol)
    print(f"  rel_inf out {e_out:.2e} final {e_fin:.2e}", flush=True)


def test_two_chunk_sizes_differ_from_one():
    # the option changes the result (the working memory really runs on its own grid)
    inp = wl.draw(1, 6, 9, 32, 1, seed=8200, dtype="f32", live=True)
    a, _ = run_gpu(inp, 1, "f32", 15, 4, eta_scale=2.0)
    b, _ = run_gpu(inp, 1, "f32", 15, 4, mem_chunk=6, eta_scale=2.0)
    assert np.max(np.abs(a - b)) > 1e-3 * np.max(np.abs(a))
