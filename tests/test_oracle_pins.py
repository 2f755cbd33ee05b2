"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test cites the passage it checks.  Page titles:
  [VH] "VisionHOPE: Visual Backbones as Self-Modifying Learning Systems"
  [VM] "VMamba: Visual State Space Model" (explainer page)
  [NL] "Nested Learning: The Illusion of Deep Learning Architectures", part 12
"""
import math
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ROUTE_BY_NAME = {"row_fwd": 0, "row_rev": 1, "col_fwd": 2, "col_rev": 3}


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _state(rng, d, n=1, scale=None, live=True):
    sd = math.sqrt(1.0 / d) if scale is None else scale
    st = {m: rng.standard_normal((n, d, d)) * sd for m in ("mem", "k", "v", "q")}
    st["eta"] = rng.standard_normal((n, 1, d)) * sd
    st["alpha"] = rng.standard_normal((n, 1, d)) * sd
    if not live:
        st["mem"][:] = 0.0
    return st


def _fro(a):
    return np.sqrt(np.sum(a * a, axis=(-2, -1)))


# --------------------------------------------------------------------------
# Route orders and merge: [VM] "Four orders give each position several views
# of the image" (printed 3x4 orders) and "Cross-merge restores positions
# before adding" (sum, identity scans give four times the input, rectangles).
# --------------------------------------------------------------------------
def test_route_orders_match_printed_3x4_example():
    seen = 0
    with open(os.path.join(GOLDEN, "cross_scan_3x4.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, *vals = line.split()
            got = oracle.route_order(3, 4, ROUTE_BY_NAME[name])
            assert got.tolist() == [int(v) for v in vals], name
            seen += 1
    assert seen == 4


@pytest.mark.parametrize("H,W", [(3, 4), (5, 2), (4, 4), (1, 7)])
def test_identity_scans_merge_to_four_times_input(H, W):
    rng = _rng(1)
    x, _ = wl.round_to_bf16(rng.standard_normal((2, H, W, 3)).astype(np.float32))
    x = x.astype(np.float64)
    routes = {r: oracle.cross_scan(x, r) for r in range(4)}
    out = oracle.cross_merge(routes, H, W)
    assert np.array_equal(out, 4.0 * x)
    for r in range(4):                      # each inverse alone restores the grid exactly
        assert np.array_equal(oracle.cross_merge({r: routes[r]}, H, W), x)


def test_route_chunk_lengths_follow_rows_and_columns():
    # [VH] Sec. 2.3 Eq. 25: W on the row-major routes, H on the column-major routes.
    assert [oracle.route_chunk(3, 5, r, 0) for r in range(4)] == [5, 5, 3, 3]
    assert [oracle.route_chunk(3, 5, r, 2) for r in range(4)] == [2, 2, 2, 2]


# --------------------------------------------------------------------------
# DGD core: [VH] Sec. 2.1.1 Eq. 4-6 / App. B.2.  With alpha = 1 the write is the
# exact minimiser of the proximal problem, found here by a linear solve.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("rows", [5, 1])
def test_retained_dgd_is_proximal_minimiser_at_alpha_one(rows):
    rng = _rng(2)
    d = 5
    for _ in range(5):
        W0 = rng.standard_normal((1, rows, d))
        k = rng.standard_normal((1, d))
        u = rng.standard_normal((1, rows))
        lam = float(rng.uniform(0.1, 3.0))
        eta = lam / (1.0 + lam * float(k[0] @ k[0]))          # Eq. 5
        g = -u                                                 # Eq. 6: the write target is u = -g
        got = oracle.retained_dgd(W0, k, g, np.array([eta]), np.array([1.0]))[0]
        # normal equations of Eq. 4: W (I + lam k k^T) = W0 + lam u k^T
        lhs = np.eye(d) + lam * np.outer(k[0], k[0])
        rhs = W0[0] + lam * np.outer(u[0], k[0])
        want = np.linalg.solve(lhs.T, rhs.T).T
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_retained_dgd_alpha_scales_the_retained_part():
    # Eq. 7: alpha multiplies only the retained memory, not the write.
    rng = _rng(3)
    d = 4
    M = rng.standard_normal((1, d, d))
    k = rng.standard_normal((1, d))
    g = rng.standard_normal((1, d))
    a, e = 0.7, 0.3
    full = oracle.retained_dgd(M, k, g, np.array([e]), np.array([a]))
    no_write = oracle.retained_dgd(M, k, np.zeros_like(g), np.array([e]), np.array([a]))
    np.testing.assert_allclose(full - no_write, -e * np.outer(g[0], k[0])[None], atol=1e-14)
    pure = oracle.retained_dgd(M, k, g, np.array([0.0]), np.array([a]))
    np.testing.assert_allclose(pure, a * M, atol=1e-15)


# --------------------------------------------------------------------------
# Step control: [VH] Sec. 2.2 Definition 1, Eq. 19-20; App. B.3 Eq. 38-41 and
# the finite-precision safeguards.
# --------------------------------------------------------------------------
def _tokens(rng, n, d, adversarial=False):
    k = oracle.stabilized_normalize(rng.standard_normal((n, d)) * rng.uniform(0.001, 3, (n, 1)))
    v = rng.standard_normal((n, d)) * rng.uniform(0.0, 2, (n, 1))
    if adversarial:
        v[: n // 2] = k[: n // 2] + 1e-9 * rng.standard_normal((n // 2, d))   # delta ~ 0
    delta = k - v
    alpha = rng.uniform(1e-3, 0.999, n)
    if adversarial:
        alpha[: n // 2] = rng.uniform(1e-4, 0.05, n // 2)
    eta = np.exp(rng.uniform(-6, 7, n))
    return k, delta, eta, alpha


def test_soft_cap_bounds_and_derivative():
    rng = _rng(4)
    k, delta, eta, alpha = _tokens(rng, 400, 8)
    eta_bar, eta_inj = oracle.soft_injection_cap(eta, alpha, delta)
    assert np.all(eta_bar > 0) and np.all(eta_bar <= eta_inj)            # 0 < eta_bar < eta_inj
    moderate = eta / eta_inj < 30.0            # beyond this 1 - exp(-x) rounds to 1 in fp64
    assert moderate.sum() > 100 and np.all(eta_bar[moderate] < eta_inj[moderate])
    # Eq. 38: d eta_bar / d eta = exp(-eta / eta_inj), by central differences
    h = 1e-6 * eta
    up, _ = oracle.soft_injection_cap(eta + h, alpha, delta)
    dn, _ = oracle.soft_injection_cap(eta - h, alpha, delta)
    fd = (up - dn) / (2 * h)
    np.testing.assert_allclose(fd, np.exp(-eta / eta_inj), rtol=1e-5, atol=1e-9)


def test_soft_cap_small_step_series():
    # Eq. 39: eta_bar = eta - eta^2 / (2 eta_inj) + O(eta^3 / eta_inj^2)
    rng = _rng(5)
    k, delta, _, alpha = _tokens(rng, 50, 6)
    _, inj = oracle.soft_injection_cap(np.ones(50), alpha, delta)
    for frac in (1e-2, 1e-3):
        eta = frac * inj
        eta_bar, _ = oracle.soft_injection_cap(eta, alpha, delta)
        err = eta_bar - (eta - eta ** 2 / (2 * inj))
        np.testing.assert_allclose(err, eta ** 3 / (6 * inj ** 2), rtol=0.02)


def test_injection_limit_uses_inward_factor_and_stabilized_norm():
    # Eq. 19 with the App. B.3 inward factor 1 - 1e-3 on the injection limit.
    delta = np.array([[3.0, 4.0]])
    _, inj = oracle.soft_injection_cap(np.array([1.0]), np.array([0.5]), delta, eps=0.0)
    assert inj[0] == pytest.approx((1 - 1e-3) * 0.5 / 5.0, rel=1e-15)


def test_spectral_clamp_and_operator_bounds():
    # Prop. 1 (Eq. 22): ||A||_2 <= alpha and ||B||_2 < 1 - alpha, by SVD, also on
    # tokens built so that the spectral clamp binds.
    rng = _rng(6)
    d = 6
    k, delta, eta, alpha = _tokens(rng, 600, d, adversarial=True)
    step = oracle.executed_step(eta, alpha, k, delta)
    eta_bar, _ = oracle.soft_injection_cap(eta, alpha, delta)
    spec = oracle.spectral_limit(alpha, k)
    assert np.all(step * np.sum(k * k, -1) <= 2 * alpha)                # Eq. 40
    assert np.all(spec < 2 * alpha / np.maximum(np.sum(k * k, -1), 1e-20))
    clamped = step < eta_bar
    assert clamped.sum() > 10                                            # the clamp does fire
    assert np.all(step[clamped] == spec[clamped])
    for i in range(len(step)):
        A = alpha[i] * np.eye(d) - step[i] * np.outer(k[i], k[i])
        B = -step[i] * np.outer(delta[i], k[i])
        assert np.linalg.norm(A, 2) <= alpha[i] * (1 + 1e-12)
        assert np.linalg.norm(B, 2) < 1 - alpha[i]
        assert np.linalg.norm(A + B, 2) < 1.0                            # Cor. 1, Eq. 43


def test_spectral_limit_rounds_toward_zero_and_floors_kappa():
    a = np.array([0.3])
    k0 = np.zeros((1, 4))
    lim = oracle.spectral_limit(a, k0)                                   # kappa floored at 1e-20
    assert lim[0] == np.nextafter((1 - 1e-6) * 2 * 0.3 / 1e-20, 0)
    lim32 = oracle.spectral_limit(a, np.full((1, 4), 0.5), dtype=np.float32)
    assert lim32[0] == float(np.nextafter(np.float32((1 - 1e-6) * 0.6), np.float32(0)))


def test_zero_step_and_unit_retention_edge_cases():
    delta = np.array([[0.3, -0.1]])
    eb, _ = oracle.soft_injection_cap(np.array([0.0]), np.array([0.9]), delta)
    assert eb[0] == 0.0
    eb, inj = oracle.soft_injection_cap(np.array([0.5]), np.array([1.0]), delta)
    assert inj[0] == 0.0 and eb[0] == 0.0


# --------------------------------------------------------------------------
# Chain-level pins.
# --------------------------------------------------------------------------
def _run_prefixes(xs, st, chunk, **kw):
    """Final states after every prefix length 0..N (same chunking)."""
    out = [oracle.flatten_state({m: st[m].copy() for m in oracle.MEMORIES})]
    for t in range(1, xs.shape[1] + 1):
        _, fin = oracle.srnl_chain(xs[:, :t], st, chunk, **kw)
        out.append(oracle.flatten_state(fin))
    return out


def test_tokenwise_run_is_non_expansive_per_memory():
    # Cor. 1 (Eq. 23): at C = 1 every memory norm is non-increasing token by token.
    rng = _rng(7)
    d, N, n = 5, 20, 3
    st = _state(rng, d, n)
    xs = rng.standard_normal((n, N, d)) * 2.0
    states = _run_prefixes(xs, st, 1, eta_scale=5.0)
    for a, b in zip(states[:-1], states[1:]):
        sa, sb = oracle.unflatten_state(a, d), oracle.unflatten_state(b, d)
        for m in oracle.MEMORIES:
            assert np.all(_fro(sb[m]) <= _fro(sa[m]) * (1 + 1e-12))


def test_uncontrolled_recurrence_can_expand():
    # Negative control for Eq. 18: with the executed step replaced by the raw step
    # the same checks fail, so the non-expansion tests have teeth.
    rng = _rng(8)
    d, N, n = 5, 12, 4
    st = _state(rng, d, n)
    xs = rng.standard_normal((n, N, d)) * 2.0
    grew = False
    prev = st
    with np.errstate(over="ignore", invalid="ignore"):
        for t in range(N):
            _, fin = oracle.srnl_chain(xs[:, t:t + 1], prev, 1, eta_scale=20.0, control=False)
            if np.any(_fro(fin["k"]) > _fro(prev["k"]) * (1 + 1e-9)):
                grew = True
                break
            prev = fin
    assert grew


def test_chunk_literal_loop_equals_shared_gain():
    # [VH] App. B.4: Eq. 45 per memory equals M_b G_t with the shared gain of
    # Eq. 46 (Prop. 2); ||G_t||_2 <= 1 and ||M_t||_F <= ||M_b||_F (Thm. 1).
    rng = _rng(9)
    d, C, n = 6, 7, 3
    st = _state(rng, d, n)
    xs = rng.standard_normal((n, C, d)) * 1.5
    log = []
    oracle.srnl_chain(xs, st, C, eta_scale=3.0, log=log)
    k = np.stack([e["k"] for e in log], 1)
    delta = np.stack([e["delta"] for e in log], 1)
    step = np.stack([e["step"] for e in log], 1)
    alpha = np.stack([e["alpha"] for e in log], 1)
    gains = oracle.chunk_gain(k, delta, step, alpha)
    prefixes = _run_prefixes(xs, st, C, eta_scale=3.0)
    for t in range(C + 1):
        fin = oracle.unflatten_state(prefixes[t], d)
        for m in oracle.MEMORIES:
            want = st[m] @ gains[t]
            np.testing.assert_allclose(fin[m], want, rtol=1e-11, atol=1e-13)
            assert np.all(_fro(fin[m]) <= _fro(st[m]) * (1 + 1e-12))
        assert np.all(np.linalg.norm(gains[t], 2, axis=(1, 2)) <= 1 + 1e-12)


def test_scalar_head_closed_form():
    # [VH] App. B.4 Eq. 49 at d = 1: G = prod A + sum_j B_j prod_{s>j} A_s, evaluated
    # as an explicit sum of products of the logged per-token scalars.
    rng = _rng(10)
    d, N, C = 1, 9, 4
    st = _state(rng, d, 2, scale=0.8)
    xs = rng.standard_normal((2, N, d))
    log = []
    ys, fin = oracle.srnl_chain(xs, st, C, eta_scale=2.0, log=log)
    for c in range(2):
        M = {m: float(st[m][c, 0, 0]) for m in oracle.MEMORIES}
        for s in range(0, N, C):
            ts = list(range(s, min(s + C, N)))
            A = [log[t]["alpha"][c] - log[t]["step"][c] * log[t]["k"][c, 0] ** 2 for t in ts]
            Bv = [-log[t]["step"][c] * log[t]["delta"][c, 0] * log[t]["k"][c, 0] for t in ts]
            G = math.prod(A) + sum(Bv[j] * math.prod(A[j + 1:]) for j in range(len(ts)))
            M = {m: M[m] * G for m in M}
        for m in oracle.MEMORIES:
            assert fin[m][c, 0, 0] == pytest.approx(M[m], rel=1e-12, abs=1e-300)


def test_zero_step_is_pure_retention_decay():
    # eta = 0 gives T_t = alpha_t I and B_t = 0 (Eq. 21): every memory is the initial
    # memory times the running product of alpha.  alpha itself comes from the decaying
    # retention memory, so the whole run reduces to a scalar recurrence.
    rng = _rng(11)
    d, N, C, n = 4, 11, 3, 2
    st = _state(rng, d, n)
    xs = rng.standard_normal((n, N, d))
    ys, fin = oracle.srnl_chain(xs, st, C, eta_scale=0.0, alpha_bias=2.0)
    for c in range(n):
        decay = 1.0
        for s in range(0, N, C):
            a_b = decay * st["alpha"][c, 0]                 # boundary retention memory
            for t in range(s, min(s + C, N)):
                decay_t = 1.0 / (1.0 + math.exp(-(float(a_b @ xs[c, t]) + 2.0)))
                if t == s:
                    chunk_prod = decay_t
                else:
                    chunk_prod *= decay_t
                # readout at the chunk start state: M_mem scaled by the decay so far
                q = decay * (st["q"][c] @ xs[c, t])
                q = q / math.sqrt(float(q @ q) + 1e-6)
                np.testing.assert_allclose(ys[c, t], decay * (st["mem"][c] @ q), rtol=1e-12)
            decay *= chunk_prod
        for m in oracle.MEMORIES:
            np.testing.assert_allclose(fin[m][c], decay * st[m][c], rtol=1e-12)


def test_initial_gates_with_zero_scalar_memories():
    # [VH] App. C.1: zero scalar memories give eta = gamma * ln 2 (softplus) or
    # eta_scale / 2 (sigmoid), and alpha = sigmoid(bias) = alpha_init.
    rng = _rng(12)
    d = 4
    st = _state(rng, d, 1)
    st["eta"][:] = 0.0
    st["alpha"][:] = 0.0
    xs = rng.standard_normal((1, 3, d))
    log = []
    oracle.srnl_chain(xs, st, 3, eta_map="softplus", eta_scale=0.025,
                      alpha_bias=math.log(0.9 / 0.1), log=log)
    for e in log:
        assert e["eta"][0] == pytest.approx(0.025 * math.log(2), rel=1e-15)
        assert e["alpha"][0] == pytest.approx(0.9, rel=1e-15)
    log = []
    oracle.srnl_chain(xs, st, 3, eta_scale=1.0, alpha_bias=4.0, log=log)
    for e in log:
        assert e["eta"][0] == 0.5
        assert e["alpha"][0] == pytest.approx(1 / (1 + math.exp(-4)), rel=1e-15)


def test_zero_content_memory_gives_zero_output():
    # Eq. 46: M^m_b = 0 is a fixed point, so every readout is exactly zero, while the
    # other memories still evolve.
    w = wl.WORKLOADS[0]
    inp = wl.draw_workload(w, live=False)
    out, fin = oracle.scan2d(inp["x"], inp["init"], w.n_heads)
    assert np.all(out == 0.0)
    d = w.d
    assert np.all(fin[..., : d * d] == 0.0)
    assert not np.allclose(fin[..., d * d:], inp["init"][None, ..., d * d:].astype(np.float64))
    live = wl.draw_workload(w, live=True)
    out, _ = oracle.scan2d(live["x"], live["init"], w.n_heads)
    assert np.abs(out).max() > 0.1


def test_single_chunk_reads_the_initial_state():
    # Eq. 15-16: inside one chunk every token is generated and read from the
    # chunk-start state, so with one chunk per route the readout ignores the updates.
    rng = _rng(13)
    d, N = 4, 6
    st = _state(rng, d, 1)
    xs = rng.standard_normal((1, N, d))
    ys, fin = oracle.srnl_chain(xs, st, N, eta_scale=2.0)
    ys_split, _ = oracle.srnl_chain(xs, st, 2, eta_scale=2.0)
    for t in range(N):
        qr = st["q"][0] @ xs[0, t]
        np.testing.assert_allclose(ys[0, t], st["mem"][0] @ (qr / math.sqrt(qr @ qr + 1e-6)),
                                   rtol=1e-13)
    assert not np.allclose(ys[0, 2:], ys_split[0, 2:])      # later chunks do see the updates


def test_resume_from_returned_state():
    # The chunk-start state is the whole carry: running rows [0, k) and then rows
    # [k, H) from the returned state equals one run (row-major forward route).
    rng = _rng(14)
    B, H, W, d = 2, 5, 3, 4
    x = rng.standard_normal((B, H, W, d))
    init = np.zeros((4, 1, 4 * d * d + 2 * d))
    init[0, 0] = rng.standard_normal(4 * d * d + 2 * d) * 0.5
    out, fin = oracle.scan2d(x, init, 1, dirs=1)
    k = 2
    out_a, fin_a = oracle.scan2d(x[:, :k], init, 1, dirs=1)
    init_b = np.zeros((B, 4, 1, 4 * d * d + 2 * d))
    init_b[:, 0] = fin_a[:, 0]
    out_b, fin_b = oracle.scan2d(x[:, k:], init_b, 1, dirs=1, init_per_image=True)
    np.testing.assert_allclose(np.concatenate([out_a, out_b], 1), out, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(fin_b[:, 0], fin[:, 0], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("H,W,chunk", [(3, 5, 0), (4, 4, 3), (2, 6, 0)])
def test_route_symmetries(H, W, chunk):
    # rot180 maps -> onto <- and down onto up; a transpose maps -> onto down and
    # <- onto up (chunk lengths swap with the axes).  A horizontal flip alone is
    # not a symmetry.
    rng = _rng(15)
    B, d, nh = 2, 3, 2
    x = rng.standard_normal((B, H, W, nh * d))
    S = 4 * d * d + 2 * d
    init = rng.standard_normal((4, nh, S)) * 0.5
    out, fin = oracle.scan2d(x, init, nh, chunk=chunk)
    x180 = x[:, ::-1, ::-1, :]
    out180, fin180 = oracle.scan2d(x180, init[[1, 0, 3, 2]], nh, chunk=chunk)
    np.testing.assert_allclose(out180, out[:, ::-1, ::-1, :], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(fin180, fin[:, [1, 0, 3, 2]])
    xt = x.transpose(0, 2, 1, 3)
    outt, fint = oracle.scan2d(xt, init[[2, 3, 0, 1]], nh, chunk=chunk)
    np.testing.assert_allclose(outt, out.transpose(0, 2, 1, 3), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(fint, fin[:, [2, 3, 0, 1]])
    xf = x[:, :, ::-1, :]
    outf, _ = oracle.scan2d(xf, init[[1, 0, 2, 3]], nh, chunk=chunk)
    assert not np.allclose(outf, out[:, :, ::-1, :])


def test_partial_last_chunk_matches_tokenwise_at_chunk_one():
    # With C = 1 every token is its own chunk: the fully token-indexed recurrence
    # ([VH] Eq. 13 with Eq. 9 and 14 read at t-1).  Splitting the sequence into two
    # calls at any point then leaves the result unchanged.
    rng = _rng(16)
    d, N = 3, 7
    st = _state(rng, d, 2)
    xs = rng.standard_normal((2, N, d))
    ys, fin = oracle.srnl_chain(xs, st, 1, eta_scale=2.0)
    y1, f1 = oracle.srnl_chain(xs[:, :4], st, 1, eta_scale=2.0)
    y2, f2 = oracle.srnl_chain(xs[:, 4:], f1, 1, eta_scale=2.0)
    np.testing.assert_allclose(np.concatenate([y1, y2], 1), ys, rtol=1e-14)
    for m in oracle.MEMORIES:
        np.testing.assert_allclose(f2[m], fin[m], rtol=1e-14)
    # and a chunk length that does not divide N (partial last chunk) splits at a
    # chunk boundary the same way
    ys3, fin3 = oracle.srnl_chain(xs, st, 3, eta_scale=2.0)
    ya, fa = oracle.srnl_chain(xs[:, :6], st, 3, eta_scale=2.0)
    yb, fb = oracle.srnl_chain(xs[:, 6:], fa, 3, eta_scale=2.0)
    np.testing.assert_allclose(np.concatenate([ya, yb], 1), ys3, rtol=1e-14)


# --------------------------------------------------------------------------
# Running-state readout: [NL] Eq. 94 reads y_t = M_memory,t-1 q_t; inside a chunk of
# [VH] Sec. 2.1.3 the memory after the chunk's earlier tokens is M^m_b G_{t-1}
# ([VH] App. B.4 Prop. 2), while q_t still comes from the chunk-start M_q.
# --------------------------------------------------------------------------
def test_running_readout_equals_gain_form():
    rng = _rng(31)
    d, C, n = 5, 9, 3
    st = _state(rng, d, n)
    xs = rng.standard_normal((n, C, d)) * 1.3
    log = []
    ys, _ = oracle.srnl_chain(xs, st, C, eta_scale=2.5, log=log, readout="running")
    k = np.stack([e["k"] for e in log], 1)
    delta = np.stack([e["delta"] for e in log], 1)
    step = np.stack([e["step"] for e in log], 1)
    alpha = np.stack([e["alpha"] for e in log], 1)
    gains = oracle.chunk_gain(k, delta, step, alpha)  # gains[t]: after t tokens
    for t in range(C):
        q = np.einsum("nij,nj->ni", st["q"], xs[:, t])
        q = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + 1e-6)
        want = np.einsum("nij,njk,nk->ni", st["mem"], gains[t], q)
        np.testing.assert_allclose(ys[:, t], want, rtol=1e-11, atol=1e-13)


def test_running_readout_is_boundary_readout_at_chunk_one():
    rng = _rng(32)
    st = _state(rng, 4, 2)
    xs = rng.standard_normal((2, 10, 4))
    yb, fb = oracle.srnl_chain(xs, st, 1, eta_scale=2.0, readout="boundary")
    yr, fr = oracle.srnl_chain(xs, st, 1, eta_scale=2.0, readout="running")
    assert np.array_equal(yb, yr)
    for m in oracle.MEMORIES:
        assert np.array_equal(fb[m], fr[m])  # the readout never feeds the state


def test_running_readout_zero_step_is_decayed_boundary_readout():
    # eta = 0: M^m_{t-1} = (prod of the chunk's earlier alphas) M^m_b, so the running
    # readout is the boundary readout scaled by that in-chunk product.
    rng = _rng(33)
    d, N, C, n = 4, 10, 4, 2
    st = _state(rng, d, n)
    xs = rng.standard_normal((n, N, d))
    log = []
    yr, _ = oracle.srnl_chain(xs, st, C, eta_scale=0.0, alpha_bias=1.0, log=log, readout="running")
    yb, _ = oracle.srnl_chain(xs, st, C, eta_scale=0.0, alpha_bias=1.0, readout="boundary")
    alpha = np.stack([e["alpha"] for e in log], 1)
    for s in range(0, N, C):
        prod = np.ones(n)
        for t in range(s, min(s + C, N)):
            np.testing.assert_allclose(yr[:, t], prod[:, None] * yb[:, t], rtol=1e-12)
            prod = prod * alpha[:, t]


# --------------------------------------------------------------------------
# Variants of [VH] Sec. 3.5 (ablations), Eq. 26 (direction scales) and App. B.5 (skip).
# --------------------------------------------------------------------------
def test_direction_scales_and_skip_compose_single_route_runs():
    # Eq. 26: Y = sum_r lambda_r * P_r^-1(Y_r), with Y_r = reads_r + s * Z_r (App. B.5).
    rng = _rng(41)
    B, H, W, D, nh = 2, 4, 5, 8, 2
    inp = wl.draw(B, H, W, D, nh, seed=41, dtype="f32", live=True)
    lam = rng.standard_normal((4, D))
    skip = rng.standard_normal(D)
    out, _ = oracle.scan2d(inp["x"], inp["init"], nh, route_scales=lam, skip=skip)
    want = np.zeros_like(out)
    for r in range(4):
        o_r, _ = oracle.scan2d(inp["x"], inp["init"], nh, dirs=1 << r)
        want += lam[r] * (o_r + skip * inp["x"])
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-14)
    base, _ = oracle.scan2d(inp["x"], inp["init"], nh)
    ones, _ = oracle.scan2d(inp["x"], inp["init"], nh, route_scales=np.ones((4, D)))
    assert np.array_equal(base, ones)


def test_hard_injection_clamp_bounds():
    # Sec. 3.5: a hard clamp at the same injection limit: eta_bar = min(eta, eta_inj).
    rng = _rng(42)
    n, d = 400, 6
    k = oracle.stabilized_normalize(rng.standard_normal((n, d)))
    delta = rng.standard_normal((n, d))
    alpha = oracle.sigmoid(rng.standard_normal(n) + 1.0)
    eta = np.exp(rng.standard_normal(n) * 2.0)
    _, inj = oracle.soft_injection_cap(eta, alpha, delta)
    step = oracle.executed_step(eta, alpha, k, delta, injection="hard", spectral="none")
    assert np.all(step <= eta) and np.all(step <= inj)
    below = eta <= inj
    assert below.any() and (~below).any()
    assert np.array_equal(step[below], eta[below]) and np.array_equal(step[~below], inj[~below])
    # the soft cap never exceeds the hard clamp (1 - e^-x <= x and <= 1)
    soft = oracle.executed_step(eta, alpha, k, delta, injection="soft", spectral="none")
    assert np.all(soft <= step * (1 + 1e-15))


def test_no_step_control_is_the_uncontrolled_recurrence():
    rng = _rng(43)
    st = _state(rng, 4, 2)
    xs = rng.standard_normal((2, 12, 4)) * 2.0
    y0, f0 = oracle.srnl_chain(xs, st, 3, eta_scale=1.0, control=False)
    y1, f1 = oracle.srnl_chain(xs, st, 3, eta_scale=1.0, injection="none", spectral="none")
    assert np.array_equal(y0, y1)
    for m in oracle.MEMORIES:
        assert np.array_equal(f0[m], f1[m])


def test_soft_spectral_cap_keeps_the_transition_non_expansive():
    # Sec. 3.5: a smooth map to the same spectral limit keeps eta_tilde <= eta_spec, so
    # ||alpha I - eta_tilde k k^T||_2 <= 1 (Eq. 20) even with no injection control; the
    # small-step series of the saturating map is eta_bar - eta_bar^2 / (2 eta_spec).
    rng = _rng(44)
    n, d = 300, 5
    k = oracle.stabilized_normalize(rng.standard_normal((n, d)) * 3.0)
    delta = rng.standard_normal((n, d))
    alpha = oracle.sigmoid(rng.standard_normal(n))
    eta = np.exp(rng.standard_normal(n) * 3.0)
    step = oracle.executed_step(eta, alpha, k, delta, injection="none", spectral="soft")
    lim = oracle.spectral_limit(alpha, k)
    assert np.all(step <= lim) and np.all(step <= eta)
    kk = np.sum(k * k, -1)
    assert np.all(np.abs(alpha - step * kk) <= 1.0 + 1e-12)
    small = 1e-4 * lim
    s_small = oracle.executed_step(small, alpha, k, delta, injection="none", spectral="soft")
    np.testing.assert_allclose(s_small, small - small ** 2 / (2 * lim), rtol=1e-8)  # next term x^2/6


def test_frozen_memories_stay_at_their_initial_value():
    # Sec. 3.5: without adaptive K/V (or dynamics) those memories stay as learned for the
    # whole image while the others evolve.  With one chunk per route every projection is
    # generated from the initial state anyway, so the outputs do not change at all.
    rng = _rng(45)
    d, N, n = 4, 12, 2
    st = _state(rng, d, n)
    xs = rng.standard_normal((n, N, d))
    for frozen in [("k", "v"), ("eta", "alpha"), ("q",)]:
        y_all, f_all = oracle.srnl_chain(xs, st, N, eta_scale=2.0)
        y_fr, f_fr = oracle.srnl_chain(xs, st, N, eta_scale=2.0, frozen=frozen)
        assert np.array_equal(y_all, y_fr)
        for m in oracle.MEMORIES:
            if m in frozen:
                assert np.array_equal(f_fr[m], st[m])
            else:
                assert np.array_equal(f_fr[m], f_all[m])
        _, f_c = oracle.srnl_chain(xs, st, 3, eta_scale=2.0, frozen=frozen)
        for m in frozen:
            assert np.array_equal(f_c[m], st[m])


def test_no_dgd_gain_is_a_sum_of_rank_one_writes():
    # Without the key-dependent correction (Sec. 3.5) every memory follows
    # M_t = alpha_t M_{t-1} - eta_t (M_b delta_t) k_t^T, so over a chunk
    # M_end = M_b (P(0,C) I - sum_j P(j+1,C) eta_j delta_j k_j^T), P = products of alpha.
    rng = _rng(46)
    d, C, n = 5, 8, 3
    st = _state(rng, d, n)
    xs = rng.standard_normal((n, C, d)) * 1.4
    log = []
    _, fin = oracle.srnl_chain(xs, st, C, eta_scale=2.0, dgd=False, log=log)
    G = np.zeros((n, d, d))
    for j in range(C):
        tail = np.prod([log[s]["alpha"] for s in range(j + 1, C)], axis=0) if j + 1 < C else np.ones(n)
        G -= (tail * log[j]["step"])[:, None, None] * (log[j]["delta"][:, :, None] * log[j]["k"][:, None, :])
    G += np.prod([e["alpha"] for e in log], axis=0)[:, None, None] * np.eye(d)
    for m in oracle.MEMORIES:
        np.testing.assert_allclose(fin[m], st[m] @ G, rtol=1e-11, atol=1e-13)


def test_shared_initial_state_is_a_broadcast_init():
    inp = wl.draw(1, 4, 4, 8, 2, seed=47, dtype="f32", live=True)
    shared = inp["init"][2]                          # [n_heads, S]
    a, fa = oracle.scan2d(inp["x"], shared, 2, shared_init=True)
    b, fb = oracle.scan2d(inp["x"], np.broadcast_to(shared, (4,) + shared.shape), 2)
    assert np.array_equal(a, b) and np.array_equal(fa, fb)


def test_clamp_counters_edge_values():
    inp = wl.draw(1, 4, 5, 8, 1, seed=48, dtype="f32", live=True)
    c0 = {}
    oracle.scan2d(inp["x"], inp["init"], 1, eta_scale=0.0, counts=c0)
    assert c0["updates"] == 4 * 20 and c0["inj"] == 0 and c0["spec"] == 0
    c1 = {}
    # a huge raw step with little retention headroom: the injection limit binds everywhere
    oracle.scan2d(inp["x"], inp["init"], 1, eta_scale=1e6, alpha_bias=6.0, counts=c1)
    assert c1["updates"] == 80 and c1["inj"] == 80


def test_fixed_query_projection_equals_generated_queries_when_they_agree():
    # App. B.5 / Eq. 14: with queries given from outside, q_t = n(queries[p_r(t)]) and M_q is
    # not a memory.  If the given queries are exactly what a frozen M_q would generate
    # (queries = x M_q^T for every head), the outputs equal the run with M_q frozen.
    inp = wl.draw(1, 4, 5, 8, 2, seed=49, dtype="f32", live=True)
    x, init = inp["x"], inp["init"]
    d = 4
    init_shared = np.broadcast_to(init[0], init.shape).copy()  # every route: route 0's memories
    q = np.concatenate([x[..., h * d:(h + 1) * d] @ oracle.unflatten_state(init[0, h], d)["q"].T
                        for h in range(2)], axis=-1)
    a, fa = oracle.scan2d(x, init_shared, 2, queries=q)
    b, fb = oracle.scan2d(x, init_shared, 2, frozen=("q",))
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(fa, fb, rtol=1e-12, atol=1e-14)
    assert np.array_equal(oracle.unflatten_state(fa[0, 3, 1], d)["q"], oracle.unflatten_state(init[0, 1], d)["q"])


# --------------------------------------------------------------------------
# Two chunk sizes ([NLz] Sec. 2.10): the working memory M_mem keeps its boundary state
# over chunks of its own length, the five projection memories over theirs.
# --------------------------------------------------------------------------
def test_two_chunk_sizes_reduce_to_one_when_equal():
    rng = _rng(71)
    st = _state(rng, 5, 2)
    xs = rng.standard_normal((2, 13, 5)) * 1.2
    for C in (1, 4, 13):
        y1, f1 = oracle.srnl_chain(xs, st, C, eta_scale=2.0)
        y2, f2 = oracle.srnl_chain(xs, st, C, eta_scale=2.0, mem_chunk=C)
        assert np.array_equal(y1, y2)
        for m in oracle.MEMORIES:
            assert np.array_equal(f1[m], f2[m])


@pytest.mark.parametrize("C,Cm", [(4, 3), (3, 5), (6, 2), (1, 4)])
def test_two_chunk_sizes_scalar_head_closed_form(C, Cm):
    # d = 1: every memory is a scalar and its chunk gain is prod A + sum_j B_j prod_{s>j} A_s
    # (Eq. 49) over the tokens of ITS chunk, from the logged per-token scalars; M_mem groups
    # the tokens by Cm, the other memories by C.  Its readout is M_mem at the start of the
    # token's Cm-chunk times q_t.
    rng = _rng(72)
    d, N = 1, 13
    st = _state(rng, d, 2, scale=0.8)
    xs = rng.standard_normal((2, N, d))
    log = []
    ys, fin = oracle.srnl_chain(xs, st, C, eta_scale=2.0, log=log, mem_chunk=Cm)
    for c in range(2):
        A = [log[t]["alpha"][c] - log[t]["step"][c] * log[t]["k"][c, 0] ** 2 for t in range(N)]
        Bv = [-log[t]["step"][c] * log[t]["delta"][c, 0] * log[t]["k"][c, 0] for t in range(N)]

        def run(m0, L, upto):
            # the memory after `upto` tokens, chunked by L, and its value at each boundary
            val, bound = m0, {}
            for s in range(0, upto, L):
                ts = list(range(s, min(s + L, upto)))
                bound[s] = val
                val *= math.prod(A[t] for t in ts) + sum(
                    Bv[j] * math.prod(A[t] for t in ts[i + 1:]) for i, j in enumerate(ts))
            return val, bound

        for m in oracle.MEMORIES:
            L = Cm if m == "mem" else C
            want, _ = run(float(st[m][c, 0, 0]), L, N)
            assert fin[m][c, 0, 0] == pytest.approx(want, rel=1e-12, abs=1e-300)
        # readout: q_t from M_q at the start of the token's C-chunk, read by M_mem at the
        # start of its Cm-chunk
        _, qb = run(float(st["q"][c, 0, 0]), C, N)
        _, mb = run(float(st["mem"][c, 0, 0]), Cm, N)
        for t in range(N):
            z = qb[(t // C) * C] * xs[c, t, 0]
            q = z / math.sqrt(z * z + 1e-6)
            assert ys[c, t, 0] == pytest.approx(mb[(t // Cm) * Cm] * q, rel=1e-12, abs=1e-300)


@pytest.mark.parametrize("C,Cm", [(3, 5), (5, 2), (4, 4)])
def test_two_chunk_sizes_zero_step_decay(C, Cm):
    # eta = 0: every memory is its initial value times the running product of alpha.  The
    # projections (so alpha and q) come from the retention and query memories at the start
    # of the token's C-chunk; the readout from M_mem at the start of its Cm-chunk.
    rng = _rng(73)
    d, N, n = 4, 13, 2
    st = _state(rng, d, n)
    xs = rng.standard_normal((n, N, d))
    ys, fin = oracle.srnl_chain(xs, st, C, eta_scale=0.0, alpha_bias=2.0, mem_chunk=Cm)
    for c in range(n):
        decay = [1.0]                                   # decay[t]: product of alpha_s, s < t
        for t in range(N):
            b = (t // C) * C
            s_a = decay[b] * float(st["alpha"][c, 0] @ xs[c, t]) + 2.0
            decay.append(decay[t] / (1.0 + math.exp(-s_a)))
        for t in range(N):
            q = decay[(t // C) * C] * (st["q"][c] @ xs[c, t])
            q = q / math.sqrt(float(q @ q) + 1e-6)
            want = decay[(t // Cm) * Cm] * (st["mem"][c] @ q)
            np.testing.assert_allclose(ys[c, t], want, rtol=1e-12)
        for m in oracle.MEMORIES:
            np.testing.assert_allclose(fin[m][c], decay[N] * st[m][c], rtol=1e-12)
