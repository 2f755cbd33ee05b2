"""fp64 CPU oracle of the VisionHOPE block around the four-direction scan.

TEST INFRASTRUCTURE ONLY, like ``hope_oracle``: only ``tests/``, ``__graft_entry__.smoke()``
and the benchmark's CPU baseline may import it; it shares no code with the HIP path.

The block ("VisionHOPE: Visual Backbones as Self-Modifying Learning Systems", Sec. 2.3
Eq. 27 and App. B.5), for a channels-last input x [B, H, W, D], inference form (no
stochastic depth):

  x1  = x + CPE(x)                            conditional positional encoding, a 3x3
                                              depthwise convolution added to its input
  u   = LN1(x1) W_in^T + b_in                 pre-normalisation, pointwise projection D -> D_m
  z   = u + SiLU(DW(u))                       the gated depthwise-convolutional residual branch
  q   = z W_q^T                               the outer query projection, shared by the routes
  y   = VH(z; queries q, skip, scales) + LPE(z)   the four-direction operator with its
                                              channel-wise skip and direction scales, plus the
                                              depthwise local positional branch on z
  x'  = x1 + y W_out^T + b_out                output projection D_m -> D, residual
  out = x' + GELU(LN2(x') W_1^T + b_1) W_2^T + b_2   the FFN branch (expansion 4), residual

The inner width D_m is whatever the weights give (w_in is [D_m, D]); the pages' evaluated
models use D_m = D / 2 with heads of 16 (App. C.3).  Readings where the pages leave the form
open (listed in the design notes as R22-R26): all depthwise convolutions are 3x3 with zero
padding and a bias; the gated branch is u + SiLU(DW(u)); LayerNorm eps 1e-5 with an affine
map; GELU is the erf form; W_q has no bias.  Linear weights are stored [out, in]
(y = x W^T + b); depthwise weights [3][3][C].

Pins: tests/test_oracle_block_pins.py.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from .hope_oracle import scan2d

LN_EPS = 1e-5


def dwconv3x3(x, w, b):
    """Depthwise 3x3 convolution with zero padding: out[y, x, c] = b[c] +
    sum over dy, dx in {-1, 0, 1} of w[dy + 1, dx + 1, c] * x[y + dy, x + dx, c]."""
    x = np.asarray(x, dtype=np.float64)
    B, H, W, C = x.shape
    xp = np.zeros((B, H + 2, W + 2, C))
    xp[:, 1:-1, 1:-1] = x
    out = np.broadcast_to(np.asarray(b, dtype=np.float64), x.shape).copy()
    for dy in range(3):
        for dx in range(3):
            out += np.asarray(w, dtype=np.float64)[dy, dx] * xp[:, dy:dy + H, dx:dx + W]
    return out


def layer_norm(x, g, b, eps: float = LN_EPS):
    """Per-pixel normalisation over channels with the biased variance, then g * . + b."""
    mu = x.mean(-1, keepdims=True)
    var = ((x - mu) ** 2).mean(-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(g, np.float64) + np.asarray(b, np.float64)


def silu(x):
    return x / (1.0 + np.exp(-x))


def gelu(x):
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def linear(x, w, b=None):
    """x [..., in] W[out, in]^T (+ b)."""
    y = x @ np.asarray(w, dtype=np.float64).T
    return y if b is None else y + np.asarray(b, dtype=np.float64)


def block_forward(x, wts: dict, n_heads: int, chunk: int = 0, return_parts: bool = False):
    """The block of Eq. 27 / App. B.5 on x [B, H, W, D] (fp64 result).  wts holds cpe_w,
    cpe_b, ln1_g, ln1_b, w_in, b_in, dw_w, dw_b, w_q, init ([4, n_heads, S]), scales
    ([4, D_m]), skip ([D_m]), lpe_w, lpe_b, w_out, b_out, ln2_g, ln2_b, w1, b1, w2, b2."""
    x = np.asarray(x, dtype=np.float64)
    x1 = x + dwconv3x3(x, wts["cpe_w"], wts["cpe_b"])
    u = linear(layer_norm(x1, wts["ln1_g"], wts["ln1_b"]), wts["w_in"], wts["b_in"])
    z = u + silu(dwconv3x3(u, wts["dw_w"], wts["dw_b"]))
    q = linear(z, wts["w_q"])
    y, _ = scan2d(z, wts["init"], n_heads, chunk=chunk, queries=q, route_scales=wts["scales"],
                  skip=wts["skip"])
    y = y + dwconv3x3(z, wts["lpe_w"], wts["lpe_b"])
    x2 = x1 + linear(y, wts["w_out"], wts["b_out"])
    h = gelu(linear(layer_norm(x2, wts["ln2_g"], wts["ln2_b"]), wts["w1"], wts["b1"]))
    out = x2 + linear(h, wts["w2"], wts["b2"])
    if return_parts:
        return out, dict(x1=x1, u=u, z=z, q=q, y=y, x2=x2, h=h)
    return out
