"""Seeded synthetic inputs for the four-direction Hope memory scan.

This module only draws numbers; it holds none of the method's arithmetic, so
both the fp64 oracle (``oracle/``) and the HIP path can be fed from it.

Shapes follow the pages' workloads (VisionHOPE, App. C.1 "Shared VisionHOPE
settings": row/column chunks equal to the feature-map width/height; VMamba
explainer, backbone stage widths 56^2x96, 28^2x192, 14^2x384).  The pages'
images and weights are not available, so the feature map is x ~ N(0, 1) and
every initial memory is N(0, 1/d_h) (d_h = head dimension).

Draw order (one numpy PCG64 stream per workload, seed = workload index):
  1. x[B, H, W, D] ~ N(0, 1)
  2. for route r in (->, <-, down, up), for head h:
       M_mem, M_k, M_v, M_q ~ N(0, 1/d) each d x d (row-major, applied as M @ x),
       m_eta, m_alpha ~ N(0, 1/d) each 1 x d
  3. the literal variant zeroes M_mem after drawing, so the "live" variant
     (M_mem kept) shares every other draw.
bf16 workloads hand the GPU the round-to-nearest-even bf16 of the fp32 draw;
the oracle receives the same rounded values widened to fp64.
"""
from __future__ import annotations

import dataclasses
import numpy as np

ROUTE_NAMES = ("row_fwd", "row_rev", "col_fwd", "col_rev")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    W: int
    D: int
    n_heads: int
    chunk: int          # 0 = aligned (W on row routes, H on column routes)
    dtype: str          # "f32" or "bf16"
    seed: int

    @property
    def d(self) -> int:
        return self.D // self.n_heads

    @property
    def state_size(self) -> int:
        d = self.d
        return 4 * d * d + 2 * d

    def scan_tokens(self, n_dirs: int = 4) -> int:
        return self.B * self.H * self.W * n_dirs

    def with_batch(self, B: int) -> "Workload":
        return dataclasses.replace(self, B=B)


WORKLOADS = [
    Workload("tiny_8x8_d16x1_c8_f32", 1, 8, 8, 16, 1, 0, "f32", 0),
    Workload("stage1_56x56_d96_3x32_c56_bf16", 16, 56, 56, 96, 3, 0, "bf16", 1),
    Workload("stage2_28x28_d192_6x32_c28_bf16", 64, 28, 28, 192, 6, 0, "bf16", 2),
    Workload("stage3_14x14_d384_6x64_c14_bf16", 128, 14, 14, 384, 6, 0, "bf16", 3),
    Workload("hires_128x128_d96_3x32_c128_bf16", 2, 128, 128, 96, 3, 0, "bf16", 4),
]

# gate constants of these workloads: eta = eta_scale * sigmoid(s), alpha = sigmoid(s + alpha_bias)
ETA_SCALE = 1.0
ALPHA_BIAS = 4.0
EPS = 1e-6


def round_to_bf16(a: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round fp32 values to bf16 (nearest, ties to even).

    Returns (values as fp32, raw bf16 bit patterns as uint16)."""
    a32 = np.ascontiguousarray(a, dtype=np.float32)
    u = a32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    u32 = u.astype(np.uint32)
    return u32.view(np.float32), (u32 >> 16).astype(np.uint16)


def draw(B: int, H: int, W: int, D: int, n_heads: int, seed: int, dtype: str = "f32",
         live: bool = False, init_per_image: bool = False, x_scale: float = 1.0,
         mem_scale: float = 1.0) -> dict:
    """Draw one synthetic workload.

    Returns a dict with
      x      : fp32 [B, H, W, D]  (values exactly representable in ``dtype``)
      x_bits : uint16 [B, H, W, D] bf16 bit patterns (bf16 only, else None)
      init   : fp32 [4, n_heads, S] or [B, 4, n_heads, S], S = 4d^2 + 2d
    """
    if D % n_heads:
        raise ValueError("D must be a multiple of n_heads")
    d = D // n_heads
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((B, H, W, D)) * x_scale
    x32 = x.astype(np.float32)
    x_bits = None
    if dtype == "bf16":
        x32, x_bits = round_to_bf16(x32)
    elif dtype != "f32":
        raise ValueError(dtype)
    sd = np.sqrt(1.0 / d) * mem_scale
    lead = (B,) if init_per_image else ()
    S = 4 * d * d + 2 * d
    init = np.empty(lead + (4, n_heads, S), dtype=np.float32)
    for r in range(4):
        for h in range(n_heads):
            mats = [rng.standard_normal(lead + (d, d)) * sd for _ in range(4)]
            rows = [rng.standard_normal(lead + (d,)) * sd for _ in range(2)]
            if not live:
                mats[0] = np.zeros_like(mats[0])
            flat = [m.reshape(lead + (d * d,)) for m in mats] + rows
            init[..., r, h, :] = np.concatenate(flat, axis=-1).astype(np.float32)
    return {"x": x32, "x_bits": x_bits, "init": init, "d": d}


def draw_workload(w: Workload, live: bool = False, B: int | None = None, seed_offset: int = 0) -> dict:
    """Draw a named workload; ``live`` keeps the drawn content memory M_mem."""
    return draw(w.B if B is None else B, w.H, w.W, w.D, w.n_heads, w.seed + seed_offset,
                w.dtype, live=live)


def split_state(flat: np.ndarray, d: int) -> dict:
    """View a flat per-(route, head) state vector [..., 4d^2+2d] as named memories.

    Pure re-indexing: M_mem, M_k, M_v, M_q as [..., d, d]; m_eta, m_alpha as [..., 1, d]."""
    dd = d * d
    out = {}
    for i, name in enumerate(("mem", "k", "v", "q")):
        out[name] = flat[..., i * dd:(i + 1) * dd].reshape(flat.shape[:-1] + (d, d))
    out["eta"] = flat[..., 4 * dd:4 * dd + d].reshape(flat.shape[:-1] + (1, d))
    out["alpha"] = flat[..., 4 * dd + d:4 * dd + 2 * d].reshape(flat.shape[:-1] + (1, d))
    return out


BLOCK_LINEAR = ("w_in", "w_q", "w_out", "w1", "w2")


def draw_block_weights(D: int, n_heads: int, ffn_dim: int, seed: int, D_m: int | None = None) -> dict:
    """Synthetic weights of one VisionHOPE block (the pages' trained weights are absent).

    D is the block width, D_m the operator's inner width (default D; the pages' evaluated
    models use D_m = D / 2 with n_heads = D / 32 heads of 16), split into n_heads heads.
    Linear weights [out, in] ~ N(0, 1/in), rounded to bf16 (values as fp32 under their
    names, bit patterns under name + "_bits"): w_in [D_m, D], w_q [D_m, D_m], w_out [D, D_m],
    w1 [ffn_dim, D], w2 [D, ffn_dim]; depthwise 3x3 weights [3, 3, C] ~ N(0, 1/9) scaled by
    0.5 (C = D for the positional encoding, D_m for the two branches inside); biases
    ~ N(0, 0.02^2); LayerNorm gains 1 + N(0, 0.1^2) and shifts N(0, 0.1^2); direction scales
    1 + N(0, 0.1^2) [4, D_m]; skip N(0, 0.1^2) [D_m]; initial memories [4, n_heads, 4d^2 + 2d]
    ~ N(0, 1/d), d = D_m / n_heads, M_mem kept.  Draw order: the names in the order listed by
    the returned dict's construction below, one PCG64 stream."""
    Dm = D if D_m is None else D_m
    d = Dm // n_heads
    rng = np.random.Generator(np.random.PCG64(seed))
    out: dict = {}

    def lin(name, n_out, n_in):
        v, bits = round_to_bf16((rng.standard_normal((n_out, n_in)) / np.sqrt(n_in)).astype(np.float32))
        out[name], out[name + "_bits"] = v, bits

    def dw(name, C):
        out[name + "_w"] = (rng.standard_normal((3, 3, C)) * (0.5 / 3.0)).astype(np.float32)
        out[name + "_b"] = (rng.standard_normal(C) * 0.02).astype(np.float32)

    def vec(name, n, mean, sd):
        out[name] = (mean + rng.standard_normal(n) * sd).astype(np.float32)

    dw("cpe", D)
    vec("ln1_g", D, 1.0, 0.1)
    vec("ln1_b", D, 0.0, 0.1)
    lin("w_in", Dm, D)
    vec("b_in", Dm, 0.0, 0.02)
    dw("dw", Dm)
    lin("w_q", Dm, Dm)
    out["scales"] = (1.0 + rng.standard_normal((4, Dm)) * 0.1).astype(np.float32)
    vec("skip", Dm, 0.0, 0.1)
    S = 4 * d * d + 2 * d
    out["init"] = (rng.standard_normal((4, n_heads, S)) / np.sqrt(d)).astype(np.float32)
    dw("lpe", Dm)
    lin("w_out", D, Dm)
    vec("b_out", D, 0.0, 0.02)
    vec("ln2_g", D, 1.0, 0.1)
    vec("ln2_b", D, 0.0, 0.1)
    lin("w1", ffn_dim, D)
    vec("b1", ffn_dim, 0.0, 0.02)
    lin("w2", D, ffn_dim)
    vec("b2", D, 0.0, 0.02)
    return out
