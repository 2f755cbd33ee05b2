"""Pins of the block oracle (oracle/hope_block.py) against things other than itself:
known values of the activations, brute-force loops on tiny inputs, shift and delta
kernels of the depthwise convolution, torch's float64 functional ops (conv2d with groups,
layer_norm, gelu, linear) for special cases of the block that reduce to them, the
identity block, and the special case that reduces to the operator oracle (itself pinned in
test_oracle_pins.py)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from oracle import hope_block as hbk


def _x(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def test_activation_known_values():
    # GELU(x) = x Phi(x): Phi(1) = 0.8413447460685429, Phi(-1) = 0.15865525393145707
    assert hbk.gelu(np.array([0.0]))[0] == 0.0
    assert hbk.gelu(np.array([1.0]))[0] == pytest.approx(0.8413447460685429, rel=1e-15)
    assert hbk.gelu(np.array([-1.0]))[0] == pytest.approx(-0.15865525393145707, rel=1e-14)
    assert hbk.gelu(np.array([30.0]))[0] == 30.0
    # SiLU(x) = x sigmoid(x): sigmoid(1) = 0.7310585786300049
    assert hbk.silu(np.array([1.0]))[0] == pytest.approx(0.7310585786300049, rel=1e-15)
    assert hbk.silu(np.array([0.0]))[0] == 0.0


def test_dwconv_brute_force_tiny():
    B, H, W, C = 1, 3, 4, 2
    x, w, b = _x((B, H, W, C), 1), _x((3, 3, C), 2), _x((C,), 3)
    got = hbk.dwconv3x3(x, w, b)
    for y in range(H):
        for xx in range(W):
            for c in range(C):
                acc = b[c]
                for dy in (-1, 0, 1):
                    for dx in (-1, 0, 1):
                        if 0 <= y + dy < H and 0 <= xx + dx < W:
                            acc += w[dy + 1, dx + 1, c] * x[0, y + dy, xx + dx, c]
                assert got[0, y, xx, c] == pytest.approx(acc, rel=1e-13, abs=1e-13)


def test_dwconv_delta_and_shift_kernels():
    x = _x((2, 5, 6, 3), 4)
    w = np.zeros((3, 3, 3))
    w[1, 1] = 1.0
    np.testing.assert_array_equal(hbk.dwconv3x3(x, w, np.zeros(3)), x)
    w = np.zeros((3, 3, 3))
    w[0, 1] = 1.0                       # out[y, x] = x[y - 1, x], zero in row 0
    s = hbk.dwconv3x3(x, w, np.zeros(3))
    np.testing.assert_array_equal(s[:, 1:], x[:, :-1])
    np.testing.assert_array_equal(s[:, 0], 0.0)


def test_dwconv_matches_torch_grouped_conv():
    import torch
    x, w, b = _x((2, 5, 7, 4), 5), _x((3, 3, 4), 6), _x((4,), 7)
    ref = torch.nn.functional.conv2d(torch.tensor(x).permute(0, 3, 1, 2),
                                     torch.tensor(w).permute(2, 0, 1)[:, None], torch.tensor(b),
                                     padding=1, groups=4).permute(0, 2, 3, 1).numpy()
    np.testing.assert_allclose(hbk.dwconv3x3(x, w, b), ref, rtol=1e-13, atol=1e-13)


def test_layer_norm_matches_torch_and_invariants():
    import torch
    x, g, b = _x((2, 3, 4, 8), 8) * 3 + 1, _x((8,), 9), _x((8,), 10)
    ref = torch.nn.functional.layer_norm(torch.tensor(x), (8,), torch.tensor(g), torch.tensor(b),
                                         eps=hbk.LN_EPS).numpy()
    np.testing.assert_allclose(hbk.layer_norm(x, g, b), ref, rtol=1e-12, atol=1e-12)
    n = hbk.layer_norm(x, np.ones(8), np.zeros(8))
    np.testing.assert_allclose(n.mean(-1), 0.0, atol=1e-13)
    var = ((x - x.mean(-1, keepdims=True)) ** 2).mean(-1)
    np.testing.assert_allclose((n ** 2).mean(-1), var / (var + hbk.LN_EPS), rtol=1e-12)


def _weights(D=16, nh=1, F=32, seed=11, Dm=None):
    w = wl.draw_block_weights(D, nh, F, seed, D_m=Dm)
    return {k: v.astype(np.float64) for k, v in w.items() if not k.endswith("_bits")}


def test_identity_block():
    # no positional encoding, zero output projection and zero FFN output: out = x exactly
    w = _weights()
    for k in ("cpe_w", "cpe_b", "w_out", "b_out", "w2", "b2"):
        w[k] = np.zeros_like(w[k])
    x = _x((1, 3, 4, 16), 12)
    np.testing.assert_array_equal(hbk.block_forward(x, w, 1), x)


def test_ffn_branch_reduces_to_torch_ops():
    # with the operator branch's output projection and the positional encoding at zero the
    # block is x + FFN(LN2(x)), computed here with torch's float64 functional ops
    import torch
    w = _weights()
    for k in ("cpe_w", "cpe_b", "w_out", "b_out"):
        w[k] = np.zeros_like(w[k])
    x = _x((1, 3, 4, 16), 13)
    F = torch.nn.functional
    t = lambda a: torch.tensor(a)
    h = F.gelu(F.linear(F.layer_norm(t(x), (16,), t(w["ln2_g"]), t(w["ln2_b"]), eps=1e-5),
                        t(w["w1"]), t(w["b1"])))
    ref = (t(x) + F.linear(h, t(w["w2"]), t(w["b2"]))).numpy()
    np.testing.assert_allclose(hbk.block_forward(x, w, 1), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("nh,Dm", [(1, 16), (2, 16), (2, 8)])
def test_operator_branch_reduces_to_the_operator_oracle(nh, Dm):
    # zero positional encodings, zero depthwise branches and a zero FFN output: out - x =
    # VH(u) W_out^T with u = LN1(x) W_in^T + b_in (torch's layer_norm and linear), the
    # operator oracle's result with the same queries, skip and scales; with D_m < D the
    # operator runs at the inner width and W_out maps it back (VisionHOPE Sec. 2.3)
    import torch
    D = 16
    w = _weights(D=D, nh=nh, Dm=Dm)
    for k in ("cpe_w", "cpe_b", "dw_w", "dw_b", "lpe_w", "lpe_b", "b_out", "w2", "b2"):
        w[k] = np.zeros_like(w[k])
    if Dm == D:
        w["w_out"] = np.eye(D)
    assert w["w_in"].shape == (Dm, D) and w["w_out"].shape == (D, Dm) and w["w_q"].shape == (Dm, Dm)
    x = _x((1, 3, 5, D), 14)
    F = torch.nn.functional
    t = lambda a: torch.tensor(a)
    u = F.linear(F.layer_norm(t(x), (D,), t(w["ln1_g"]), t(w["ln1_b"]), eps=1e-5),
                 t(w["w_in"]), t(w["b_in"])).numpy()
    q = F.linear(t(u), t(w["w_q"])).numpy()
    y, _ = oracle.scan2d(u, w["init"], nh, queries=q, route_scales=w["scales"], skip=w["skip"])
    ref = F.linear(t(y), t(w["w_out"])).numpy()
    got = hbk.block_forward(x, w, nh) - x
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def _torch_dw(a, w, b):
    import torch
    C = a.shape[-1]
    return torch.nn.functional.conv2d(torch.tensor(a).permute(0, 3, 1, 2),
                                      torch.tensor(w).permute(2, 0, 1)[:, None], torch.tensor(b),
                                      padding=1, groups=C).permute(0, 2, 3, 1).numpy()


def test_positional_encoding_branch():
    # zero output projection and zero FFN output: out = x + CPE(x) (torch grouped conv)
    w = _weights()
    for k in ("w_out", "b_out", "w2", "b2"):
        w[k] = np.zeros_like(w[k])
    x = _x((2, 4, 3, 16), 15)
    np.testing.assert_allclose(hbk.block_forward(x, w, 1), x + _torch_dw(x, w["cpe_w"], w["cpe_b"]),
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Dm", [16, 8])
def test_gated_and_local_positional_branches(Dm):
    # zero FFN output, zero CPE: out - x = (VH(z) + LPE(z)) W_out^T with z = u + SiLU(DW(u)),
    # the convolutions, SiLU and projections from torch
    import torch
    D = 16
    w = _weights(D=D, nh=2, seed=17, Dm=Dm)
    for k in ("cpe_w", "cpe_b", "b_out", "w2", "b2"):
        w[k] = np.zeros_like(w[k])
    x = _x((1, 4, 5, D), 16)
    F = torch.nn.functional
    t = lambda a: torch.tensor(a)
    u = F.linear(F.layer_norm(t(x), (D,), t(w["ln1_g"]), t(w["ln1_b"]), eps=1e-5),
                 t(w["w_in"]), t(w["b_in"])).numpy()
    z = u + F.silu(t(_torch_dw(u, w["dw_w"], w["dw_b"]))).numpy()
    q = F.linear(t(z), t(w["w_q"])).numpy()
    y, _ = oracle.scan2d(z, w["init"], 2, queries=q, route_scales=w["scales"], skip=w["skip"])
    ref = F.linear(t(y + _torch_dw(z, w["lpe_w"], w["lpe_b"])), t(w["w_out"])).numpy()
    np.testing.assert_allclose(hbk.block_forward(x, w, 2) - x, ref, rtol=1e-10, atol=1e-12)
