"""Pins of the gradient oracle (oracle/hope_backward.py) against things other than itself:

* its torch forward reproduces the numpy forward of oracle.scan2d;
* directional derivatives match central finite differences of the numpy forward, for
  the input map and the initial memories, with the step controls active;
* the content memory enters the output linearly (M_mem,t = M_mem,b G_t and G does not
  depend on M_mem), so its gradient is exactly <grad_out, out(M_mem,0 = E_ij)>, the
  output with that memory set to a basis matrix and every other memory unchanged (for the
  boundary and the running readout alike).
"""
import numpy as np
import pytest

import oracle
from oracle import hope_backward as hb

CASES = {
    # B, H, W, D, nh, chunk, options
    "aligned_sigmoid": (1, 3, 4, 8, 2, 0, dict(eta_scale=2.0)),
    "chunk5_softplus": (2, 4, 3, 4, 1, 5, dict(eta_map="softplus", eta_scale=0.5, alpha_bias=1.0)),
    "clamps": (1, 3, 3, 6, 1, 2, dict(eta_scale=40.0, alpha_bias=-1.0)),
    "scalar_heads": (1, 3, 3, 2, 2, 0, dict(eta_scale=3.0)),
    # the running readout ([VH] Sec. 2.2 reading of the memory as updated token by token)
    "running_aligned": (1, 3, 4, 8, 2, 0, dict(eta_scale=2.0, readout="running")),
    "running_chunk5_softplus": (2, 4, 3, 4, 1, 5, dict(eta_map="softplus", eta_scale=0.5, alpha_bias=1.0,
                                                       readout="running")),
    "running_clamps": (1, 3, 3, 6, 1, 2, dict(eta_scale=40.0, alpha_bias=-1.0, readout="running")),
}


def _draw(B, H, W, D, nh, seed, per_image=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    d = D // nh
    S = 4 * d * d + 2 * d
    x = rng.standard_normal((B, H, W, D))
    shape = (B, 4, nh, S) if per_image else (4, nh, S)
    init = rng.standard_normal(shape) / np.sqrt(d)
    g = rng.standard_normal((B, H, W, D))
    return x, init, g


@pytest.mark.parametrize("name", list(CASES))
def test_torch_forward_matches_numpy_forward(name):
    import torch
    B, H, W, D, nh, chunk, kw = CASES[name]
    x, init, _ = _draw(B, H, W, D, nh, 1)
    ref, _ = oracle.scan2d(x, init, nh, chunk=chunk, **kw)
    got = hb.scan2d_torch(torch.tensor(x), torch.tensor(init), nh, chunk=chunk, **kw).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("name", list(CASES))
def test_gradients_match_central_differences(name):
    B, H, W, D, nh, chunk, kw = CASES[name]
    x, init, g = _draw(B, H, W, D, nh, 2)
    gx, gi = hb.scan2d_backward(x, init, nh, g, chunk=chunk, **kw)

    def f(xx, ii):
        out, _ = oracle.scan2d(xx, ii, nh, chunk=chunk, **kw)
        return float(np.sum(out * g))

    rng = np.random.Generator(np.random.PCG64(3))
    h = 1e-6
    for _ in range(3):
        vx = rng.standard_normal(x.shape)
        vi = rng.standard_normal(init.shape)
        fd_x = (f(x + h * vx, init) - f(x - h * vx, init)) / (2 * h)
        fd_i = (f(x, init + h * vi) - f(x, init - h * vi)) / (2 * h)
        assert np.sum(gx * vx) == pytest.approx(fd_x, rel=2e-6, abs=1e-7)
        assert np.sum(gi * vi) == pytest.approx(fd_i, rel=2e-6, abs=1e-7)


def test_gradients_per_image_initial_state():
    B, H, W, D, nh = 2, 3, 3, 4, 1
    x, init, g = _draw(B, H, W, D, nh, 4, per_image=True)
    _, gi = hb.scan2d_backward(x, init, nh, g, chunk=2, eta_scale=2.0, init_per_image=True)
    _, gshared = hb.scan2d_backward(x[:1], init[0], nh, g[:1], chunk=2, eta_scale=2.0)
    # image 0's gradient with its own initial state equals the shared-state gradient of a
    # one-image batch
    np.testing.assert_allclose(gi[0], gshared, rtol=1e-12, atol=1e-14)
    h = 1e-6
    v = np.random.Generator(np.random.PCG64(5)).standard_normal(init.shape)

    def f(ii):
        out, _ = oracle.scan2d(x, ii, nh, chunk=2, eta_scale=2.0, init_per_image=True)
        return float(np.sum(out * g))
    fd = (f(init + h * v) - f(init - h * v)) / (2 * h)
    assert np.sum(gi * v) == pytest.approx(fd, rel=2e-6, abs=1e-7)


@pytest.mark.parametrize("name", ["aligned_sigmoid", "clamps", "running_clamps"])
def test_content_memory_gradient_is_exact_linear_response(name):
    B, H, W, D, nh, chunk, kw = CASES[name]
    x, init, g = _draw(B, H, W, D, nh, 6)
    _, gi = hb.scan2d_backward(x, init, nh, g, chunk=chunk, **kw)
    d = D // nh
    for r in range(4):
        for h in range(nh):
            for i in range(d):
                for j in range(d):
                    basis = init.copy()
                    basis[r, h, :d * d] = 0.0
                    basis[r, h, i * d + j] = 1.0
                    # only route r, head h reads this memory: the other routes / heads
                    # contribute the same to both runs, so take the difference
                    zero = init.copy()
                    zero[r, h, :d * d] = 0.0
                    out1, _ = oracle.scan2d(x, basis, nh, chunk=chunk, **kw)
                    out0, _ = oracle.scan2d(x, zero, nh, chunk=chunk, **kw)
                    want = float(np.sum((out1 - out0) * g))
                    assert gi[r, h, i * d + j] == pytest.approx(want, rel=1e-10, abs=1e-12)
