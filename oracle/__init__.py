"""fp64 CPU oracle of the four-direction Hope memory scan (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package; the HIP product path never does.
"""
from .hope_oracle import (  # noqa: F401
    MEMORIES, ROUTES, route_order, route_chunk, cross_scan, cross_merge, sigmoid, phi_eta,
    phi_alpha, stabilized_normalize, soft_injection_cap, spectral_limit, executed_step,
    retained_dgd, srnl_chain, scan2d, unflatten_state, flatten_state, chunk_gain,
)
