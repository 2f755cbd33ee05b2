"""Brute force on 4x4 maps: the vectorised fp64 oracle against a 50-digit mpmath
evaluation of the same equations, written with explicit index loops.

Equations: "VisionHOPE: Visual Backbones as Self-Modifying Learning Systems",
Sec. 2.1.3 Eq. 15-16 (chunk-start generation and readout), Sec. 2.2 Eq. 19-20
(step control), Sec. 2.1.2 Eq. 13 (update of every memory), Sec. 2.3 Eq. 24-26
(routes, aligned chunks, restore and sum); route orders from "VMamba: Visual
State Space Model" (the printed orders).  This catches batching mistakes (a wrong
axis, a transposed operand) that the invariants alone might let through.
"""
import numpy as np
import pytest

mp = pytest.importorskip("mpmath")

import oracle  # noqa: E402

mp.mp.dps = 50
NAMES = ("mem", "k", "v", "q", "eta", "alpha")


def _mpmat(a):
    return [[mp.mpf(float(v)) for v in row] for row in np.atleast_2d(a)]


def _mv(M, x):
    return [mp.fsum(M[i][j] * x[j] for j in range(len(x))) for i in range(len(M))]


def _normalize(z):
    n = mp.sqrt(mp.fsum(v * v for v in z) + mp.mpf("1e-6"))
    return [v / n for v in z]


def mp_chain(xs, st, C, eta_scale, alpha_bias, running=False):
    N, d = len(xs), len(xs[0])
    M = {m: [row[:] for row in st[m]] for m in NAMES}
    ys = []
    eps = mp.mpf("1e-6")
    for s in range(0, N, C):
        Mb = {m: [row[:] for row in M[m]] for m in NAMES}
        for t in range(s, min(s + C, N)):
            x = xs[t]
            k = _normalize(_mv(Mb["k"], x))
            v = _mv(Mb["v"], x)
            q = _normalize(_mv(Mb["q"], x))
            eta = eta_scale / (1 + mp.exp(-_mv(Mb["eta"], x)[0]))
            alpha = 1 / (1 + mp.exp(-(_mv(Mb["alpha"], x)[0] + alpha_bias)))
            ys.append(_mv(M["mem"] if running else Mb["mem"], q))
            delta = [k[i] - v[i] for i in range(d)]
            r = mp.sqrt(mp.fsum(z * z for z in delta) + eps * eps) + eps
            inj = (1 - mp.mpf("1e-3")) * (1 - alpha) / r
            bar = inj * (1 - mp.exp(-eta / inj))
            kappa = max(mp.fsum(z * z for z in k), mp.mpf("1e-20"))
            step = min(bar, (1 - mp.mpf("1e-6")) * 2 * alpha / kappa)
            for m in NAMES:
                resp = _mv(Mb[m], k)
                target = _mv(Mb[m], v)
                old = M[m]
                rows = len(old)
                new = [[None] * d for _ in range(rows)]
                for i in range(rows):
                    g = resp[i] - target[i]
                    for j in range(d):
                        acc = mp.fsum(old[i][l] * ((alpha if l == j else 0) - step * k[l] * k[j])
                                      for l in range(d))
                        new[i][j] = acc - step * g * k[j]
                M[m] = new
    return ys, M


@pytest.mark.parametrize("readout", ["boundary", "running"])
@pytest.mark.parametrize("d", [1, 2, 4])
@pytest.mark.parametrize("C", [1, 2, 4, 0])
def test_oracle_matches_50_digit_evaluation_on_4x4(d, C, readout):
    rng = np.random.Generator(np.random.PCG64(100 + d * 10 + C))
    H = W = 4
    B = 1
    x = rng.standard_normal((B, H, W, d))
    S = 4 * d * d + 2 * d
    init = rng.standard_normal((4, 1, S)) * np.sqrt(1.0 / d)
    eta_scale, alpha_bias = 2.0, 1.5
    out, fin = oracle.scan2d(x, init, 1, dirs=15, chunk=C, eta_scale=eta_scale,
                             alpha_bias=alpha_bias, readout=readout)
    want_out = [[[mp.mpf(0)] * d for _ in range(W)] for _ in range(H)]
    for r in range(4):
        order = oracle.route_order(H, W, r)
        xs = [[mp.mpf(float(v)) for v in x[0].reshape(H * W, d)[p]] for p in order]
        st0 = oracle.unflatten_state(init[r, 0], d)
        st = {m: _mpmat(st0[m]) for m in NAMES}
        Cr = C if C > 0 else (W if r < 2 else H)
        ys, M = mp_chain(xs, st, Cr, mp.mpf(eta_scale), mp.mpf(alpha_bias),
                         running=readout == "running")
        for t, p in enumerate(order):
            for i in range(d):
                want_out[p // W][p % W][i] += ys[t][i]
        got = oracle.unflatten_state(fin[0, r, 0], d)
        for m in NAMES:
            ref = np.array([[float(v) for v in row] for row in M[m]])
            np.testing.assert_allclose(got[m].reshape(ref.shape), ref, rtol=1e-11, atol=1e-14)
    ref_out = np.array([[[float(v) for v in px] for px in row] for row in want_out])
    np.testing.assert_allclose(out[0], ref_out, rtol=1e-11, atol=1e-14)
