"""fp64 CPU oracle of the gradients of the four-direction Hope memory scan.

TEST INFRASTRUCTURE ONLY, like ``hope_oracle``: only ``tests/`` may import it, and it
shares no code with the HIP path.

The pages call the memory trajectory explicit and differentiable ([VH] Sec. 1, the
outer gradients of the memories' initial states and of the inputs flow through every
chunk).  The gradient that the backward pass must produce is therefore the derivative
of the forward operator itself.  This module restates the forward of
``hope_oracle.srnl_chain`` / ``scan2d`` step for step in PyTorch float64 operations
(same order, same formulas; the boundary and the running readout, the two gate maps, the
default step controls) and differentiates it with ``torch.autograd``: the exact derivative of that
composition.  Its agreement with the numpy forward and with central finite differences
of the numpy oracle is pinned in ``tests/test_oracle_backward_pins.py``.

Conventions where the forward is not differentiable (measure-zero sets):
  * eta_tilde = min(eta_bar, eta_spec): the derivative follows eta_bar when
    eta_bar <= eta_spec, else eta_spec;
  * max(|k|^2, 1e-20): no derivative through the floor when it binds;
  * the one-ulp rounding of eta_spec toward zero: the value is rounded, the derivative
    is that of the unrounded limit;
  * eta_bar = 0 where eta = 0 or eta_inj = 0: derivative zero there.
"""
from __future__ import annotations

import numpy as np
import torch

from .hope_oracle import (INJ_INWARD, KAPPA_FLOOR, MEMORIES, NORM_EPS, ROUTES, SPEC_INWARD,
                          route_chunk, route_order)

_T = torch.float64


def _mv(M, x):
    """[n, rows, d] @ [n, d] -> [n, rows]."""
    return (M @ x[:, :, None])[:, :, 0]


def _normalize(z, eps):
    # [VH] App. C.1: z / sqrt(|z|^2 + eps)
    return z / torch.sqrt((z * z).sum(-1, keepdim=True) + eps)


def _phi_eta(s, eta_map, eta_scale):
    # [VH] App. C.1 Eq. 53 (softplus) or the sigmoid map of the synthetic workloads
    if eta_map == "sigmoid":
        return eta_scale * torch.sigmoid(s)
    if eta_map == "softplus":
        return eta_scale * torch.nn.functional.softplus(s)
    raise ValueError(eta_map)


def _executed_step(eta, alpha, k, delta, eps):
    # [VH] Sec. 2.2 Eq. 19-20 with the App. B.3 safeguards (soft injection cap, clamp)
    r = torch.sqrt((delta * delta).sum(-1) + eps * eps) + eps
    eta_inj = INJ_INWARD * (1.0 - alpha) / r
    ok = (eta != 0.0) & (eta_inj != 0.0)
    safe_inj = torch.where(ok, eta_inj, torch.ones_like(eta_inj))
    safe_eta = torch.where(ok, eta, torch.zeros_like(eta))
    eta_bar = torch.where(ok, safe_inj * -torch.expm1(-safe_eta / safe_inj), torch.zeros_like(eta))
    kk = (k * k).sum(-1)
    kappa = torch.where(kk > KAPPA_FLOOR, kk, torch.full_like(kk, KAPPA_FLOOR))
    lim = SPEC_INWARD * 2.0 * alpha / kappa
    lim_rounded = torch.nextafter(lim.detach(), torch.zeros_like(lim))
    lim = lim + (lim_rounded - lim.detach())          # rounded value, unrounded derivative
    return torch.where(eta_bar <= lim, eta_bar, lim)


def _chain(xs, st, chunk, eta_map, eta_scale, alpha_bias, eps, readout="boundary"):
    """srnl_chain (default controls) in torch fp64: xs [n, N, d], st name -> [n, rows, d];
    returns ys [n, N, d].  readout "boundary" reads the chunk-start memory, "running" the
    memory as updated by every earlier token."""
    n, N, d = xs.shape
    M = dict(st)
    eye = torch.eye(d, dtype=_T)
    ys = []
    for s in range(0, N, chunk):
        Mb = dict(M)                                            # [VH] Eq. 15-16: frozen at the chunk start
        for t in range(s, min(s + chunk, N)):
            x = xs[:, t, :]
            k = _normalize(_mv(Mb["k"], x), eps)
            v = _mv(Mb["v"], x)
            q = _normalize(_mv(Mb["q"], x), eps)
            eta = _phi_eta(_mv(Mb["eta"], x)[:, 0], eta_map, eta_scale)
            alpha = torch.sigmoid(_mv(Mb["alpha"], x)[:, 0] + alpha_bias)
            # y_t = M^m_b q_t, or M^m_{t-1} q_t (running: M not yet updated by token t)
            ys.append(_mv(Mb["mem"] if readout == "boundary" else M["mem"], q))
            delta = k - v
            step = _executed_step(eta, alpha, k, delta, eps)
            A = alpha[:, None, None] * eye - step[:, None, None] * (k[:, :, None] * k[:, None, :])
            for m in MEMORIES:                                  # [VH] Eq. 13 with the signal of Eq. 16
                g = _mv(Mb[m], k) - _mv(Mb[m], v)
                M[m] = M[m] @ A - step[:, None, None] * (g[:, :, None] * k[:, None, :])
    return torch.stack(ys, 1)


def _unflatten(flat, d):
    dd = d * d
    st = {}
    for i, m in enumerate(("mem", "k", "v", "q")):
        st[m] = flat[..., i * dd:(i + 1) * dd].reshape(flat.shape[:-1] + (d, d))
    st["eta"] = flat[..., 4 * dd:4 * dd + d].reshape(flat.shape[:-1] + (1, d))
    st["alpha"] = flat[..., 4 * dd + d:].reshape(flat.shape[:-1] + (1, d))
    return st


def scan2d_torch(x, init, n_heads: int, dirs: int = 15, chunk: int = 0, eta_map: str = "sigmoid",
                 eta_scale: float = 1.0, alpha_bias: float = 4.0, eps: float = NORM_EPS,
                 init_per_image: bool = False, readout: str = "boundary"):
    """The whole operator of ``hope_oracle.scan2d`` in torch fp64 (x, init: fp64 tensors)."""
    B, H, W, D = x.shape
    d = D // n_heads
    N = H * W
    out = torch.zeros((B, N, D), dtype=_T)
    flat_x = x.reshape(B, N, D)
    for h in range(n_heads):
        for r in ROUTES:                                        # fixed merge order ->, <-, down, up
            if not (dirs >> r) & 1:
                continue
            order = torch.as_tensor(route_order(H, W, r))
            xs = flat_x[:, order, h * d:(h + 1) * d]           # cross-scan ([VH] Eq. 24)
            flat = init[:, r, h] if init_per_image else init[r, h].expand(B, -1)
            st = _unflatten(flat, d)
            ys = _chain(xs, st, route_chunk(H, W, r, chunk), eta_map, eta_scale, alpha_bias, eps, readout)
            pad = torch.zeros((B, N, D), dtype=_T)
            pad[:, :, h * d:(h + 1) * d] = pad[:, :, h * d:(h + 1) * d].index_add(1, order, ys)
            out = out + pad                                     # cross-merge ([VH] Eq. 26)
    return out.reshape(B, H, W, D)


def scan2d_backward(x, init, n_heads: int, grad_out, dirs: int = 15, chunk: int = 0,
                    eta_map: str = "sigmoid", eta_scale: float = 1.0, alpha_bias: float = 4.0,
                    eps: float = NORM_EPS, init_per_image: bool = False, readout: str = "boundary"):
    """Gradients of sum(grad_out * scan2d(x, init)) with respect to x [B, H, W, D] and
    init ([4, n_heads, S], or [B, 4, n_heads, S] with init_per_image); fp64 numpy arrays."""
    xt = torch.tensor(np.asarray(x, dtype=np.float64), dtype=_T, requires_grad=True)
    it = torch.tensor(np.asarray(init, dtype=np.float64), dtype=_T, requires_grad=True)
    go = torch.tensor(np.asarray(grad_out, dtype=np.float64), dtype=_T)
    out = scan2d_torch(xt, it, n_heads, dirs, chunk, eta_map, eta_scale, alpha_bias, eps, init_per_image,
                       readout)
    (out * go).sum().backward()
    return xt.grad.numpy(), it.grad.numpy()
