"""Pins of the oracle's executed-step map (the optional step_map output of
hope_oracle.scan2d): the per-pixel executed step eta_tilde of "VisionHOPE: Visual Backbones as
Self-Modifying Learning Systems", Sec. 2.2 Eq. 19-20, indexed by route and head.

Independent checks, none of which calls the oracle's step controls:
  * small-step limit: both controls are the identity to first order as eta -> 0 (the soft
    injection cap of Eq. 19 is eta (1 - eta / (2 eta_inj) + ...), and the spectral clamp does
    not bind), so in the first chunk of every route, where the gate row is still the initial
    m_eta, eta_tilde equals eta_scale * sigmoid(m_eta . x_t) computed from the input directly;
    a wrong pixel, route, head or token in the map fails this;
  * with the controls binding (large eta, low retention) every first-chunk step lies in
    (0, eta] and some lie well below eta;
  * unselected routes are left untouched.
"""
import numpy as np

import oracle
import workloads as wl

H, W, D, NH = 3, 4, 32, 2
d = D // NH


def _first_chunk_raw_eta(inp, eta_scale):
    """eta_scale * sigmoid(m_eta . x_t) per (image, route, head, pixel) for the tokens of
    each route's first chunk (chunk = 0: W tokens on row routes, H on column routes);
    NaN elsewhere."""
    x = inp["x"].astype(np.float64)
    init = inp["init"].astype(np.float64)
    B = x.shape[0]
    out = np.full((B, 4, NH, H, W), np.nan)
    for r in range(4):
        C = W if r < 2 else H
        order = oracle.route_order(H, W, r)
        for h in range(NH):
            m_eta = init[r, h, 4 * d * d:4 * d * d + d]
            for t in range(C):
                pix = order[t]
                xt = x[:, pix // W, pix % W, h * d:(h + 1) * d]
                s = xt @ m_eta
                out[:, r, h, pix // W, pix % W] = eta_scale / (1.0 + np.exp(-s))
    return out


def test_step_map_small_step_limit():
    inp = wl.draw(2, H, W, D, NH, seed=41, live=True)
    scale = 1e-7
    sm = np.full((2, 4, NH, H, W), np.nan)
    oracle.scan2d(inp["x"], inp["init"], NH, eta_scale=scale, step_map=sm)
    assert np.all(np.isfinite(sm))
    raw = _first_chunk_raw_eta(inp, scale)
    m = np.isfinite(raw)
    assert m.sum() == 2 * NH * (2 * W + 2 * H)
    np.testing.assert_allclose(sm[m], raw[m], rtol=1e-4, atol=0)


def test_step_map_controls_bind_below_raw_eta():
    inp = wl.draw(1, H, W, D, NH, seed=43, live=True)
    scale = 50.0
    sm = np.full((1, 4, NH, H, W), np.nan)
    oracle.scan2d(inp["x"], inp["init"], NH, eta_scale=scale, alpha_bias=-3.0, step_map=sm)
    raw = _first_chunk_raw_eta(inp, scale)
    m = np.isfinite(raw)
    assert np.all(sm[m] > 0.0) and np.all(sm[m] <= raw[m] * (1 + 1e-12))
    assert np.mean(sm[m] < 0.9 * raw[m]) > 0.5


def test_step_map_leaves_unselected_routes():
    inp = wl.draw(1, H, W, D, NH, seed=45, live=True)
    sm = np.full((1, 4, NH, H, W), np.nan)
    oracle.scan2d(inp["x"], inp["init"], NH, dirs=0b0101, step_map=sm)
    assert np.all(np.isfinite(sm[:, [0, 2]])) and np.all(np.isnan(sm[:, [1, 3]]))


def test_norm_log_pure_decay_keeps_norm_ratios():
    # eta = 0 (eta_scale 0): every memory only decays, M <- alpha_t M, by the same factor per
    # token ([VH] Eq. 13 with a zero step), so the per-chunk Frobenius norms of any two
    # memories keep their initial ratio, and each chunk's norms shrink
    inp = wl.draw(2, H, W, D, NH, seed=47, live=True)
    d0 = D // NH
    xs = oracle.cross_scan(inp["x"][..., :d0].astype(np.float64), 0)
    st = oracle.unflatten_state(np.broadcast_to(inp["init"][0, 0], (2, 4 * d0 * d0 + 2 * d0)), d0)
    log = []
    oracle.srnl_chain(xs, st, W, eta_scale=0.0, norm_log=log)
    assert [e["end"] for e in log] == [W * (i + 1) for i in range(H)]
    n0 = {m: np.sqrt(np.sum(st[m] ** 2, axis=(1, 2))) for m in oracle.MEMORIES}
    prev = n0["k"]
    for e in log:
        for m in oracle.MEMORIES:
            np.testing.assert_allclose(e[m] / e["k"], n0[m] / n0["k"], rtol=1e-12)
        assert np.all(e["k"] < prev)
        prev = e["k"]
