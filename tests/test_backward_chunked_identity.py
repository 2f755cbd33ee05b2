"""The algebra of the chunk-parallel backward kernels (backward_wy.hip, and its blocked form
in backward_wy32.hip), restated in float64 and checked against the gradient oracle (oracle/hope_backward.py, itself pinned by finite
differences in test_oracle_backward_pins.py).

Two identities carry the kernel ("VisionHOPE: Visual Backbones as Self-Modifying Learning
Systems", App. B.4 Eq. 46: the six memories share the chunk's right-multiplying gain):
  * the boundary state of chunk c is S_0 P_c with P_c = G_0 ... G_{c-1}, so the reverse
    sweep carries the d x d adjoint of P instead of the (4d+2) x d state adjoint;
  * inside a chunk G_{t-1} = Gam_{t-1} I + sum_{j<t} beta_{j,t-1} u_j k_j^T and the gain
    adjoint dG_t = Gam'_t D_e - sum_{m>t} beta_{t,m-1} step_m a_m k_m^T, so every per-token
    adjoint follows from two C x C triangular recurrences and C x C Gram matrices.
This is a check of the derivation, not a second oracle: the GPU kernel is compared with
the oracle directly in test_gpu_backward.py.
"""
import numpy as np
import pytest
import torch

from oracle import hope_backward as hb
from oracle.hope_oracle import route_chunk, route_order


def gates_t(p, d, eta_scale, alpha_bias, eps, eta_map="sigmoid"):
    # p: [NP] torch -> k, delta, step, alpha, q
    kr, vr, qr, se, sa = p[:d], p[d:2*d], p[2*d:3*d], p[3*d], p[3*d+1]
    k = kr / torch.sqrt((kr*kr).sum() + eps); q = qr / torch.sqrt((qr*qr).sum() + eps)
    eta = hb._phi_eta(se, eta_map, eta_scale); alpha = torch.sigmoid(sa + alpha_bias)
    delta = k - vr
    step = hb._executed_step(eta[None], alpha[None], k[None], delta[None], eps)[0]
    return k, delta, step, alpha, q

def chain(xs, S0, dys, C, eta_scale=1.0, alpha_bias=4.0, eps=1e-6, eta_map="sigmoid"):
    N, d = xs.shape; R = S0.shape[0]
    nck = (N + C - 1) // C
    I = np.eye(d)
    def chunk_fwd(P, s0, s1):
        X = xs[s0:s1].T                      # d x c
        Xt = P @ X
        Proj = S0[d:] @ Xt                   # NP x c
        c = s1 - s0
        K = np.zeros((d, c)); Dl = np.zeros((d, c)); Q = np.zeros((d, c)); st = np.zeros(c); al = np.zeros(c)
        for t in range(c):
            k, dl, s, a, q = gates_t(torch.tensor(Proj[:, t]), d, eta_scale, alpha_bias, eps, eta_map)
            K[:, t], Dl[:, t], Q[:, t], st[t], al[t] = k.numpy(), dl.numpy(), q.numpy(), float(s), float(a)
        Gm = K.T @ K
        U = np.zeros((d, c)); Wm = np.zeros((d, c))
        gam = 1.0
        for t in range(c):
            acc = gam * K[:, t] + Dl[:, t]
            coef = 1.0
            for j in range(t - 1, -1, -1):
                acc = acc + coef * Gm[j, t] * U[:, j]
                coef *= al[j]
            Wm[:, t] = acc; U[:, t] = -st[t] * acc
            gam *= al[t]
        return X, Xt, Proj, K, Dl, Q, st, al, Gm, U, Wm
    def beta(al, j, t):  # prod_{i=j+1..t} al_i
        return float(np.prod(al[j + 1:t + 1]))
    # forward sweep
    P = I.copy(); Ps = []
    for c in range(nck):
        s0, s1 = c * C, min(N, (c + 1) * C)
        Ps.append(P.copy())
        X, Xt, Proj, K, Dl, Q, st, al, Gm, U, Wm = chunk_fwd(P, s0, s1)
        cl = s1 - s0
        bC = np.array([beta(al, j, cl - 1) for j in range(cl)])
        P = np.prod(al) * P + (P @ U) @ np.diag(bC) @ K.T
    dP = np.zeros((d, d)); dS0 = np.zeros_like(S0); dxs = np.zeros_like(xs)
    for c in range(nck - 1, -1, -1):
        s0, s1 = c * C, min(N, (c + 1) * C); cl = s1 - s0
        P = Ps[c]
        X, Xt, Proj, K, Dl, Q, st, al, Gm, U, Wm = chunk_fwd(P, s0, s1)
        Gam = np.array([np.prod(al[:t]) for t in range(cl)])            # Gamma_{t-1}
        Gp = np.array([np.prod(al[t + 1:]) for t in range(cl)])         # Gamma'_t
        Z = dP @ K; E = P.T @ Z; Y = P @ Wm; F = dP.T @ Y; trD = np.sum(P * dP)
        PU = P @ U; ud = np.sum(PU * Z, 0)
        A = np.zeros((d, cl))
        for t in range(cl - 1, -1, -1):
            acc = Gp[t] * E[:, t]
            coef = 1.0
            for m in range(t + 1, cl):
                acc = acc - coef * st[m] * Gm[m, t] * A[:, m]
                coef *= al[m]
            A[:, t] = acc
        H = U.T @ A; J = A.T @ Wm; L = np.sum(K * A, 0)
        dkg = np.zeros((d, cl)); ddl = np.zeros((d, cl)); dst = np.zeros(cl); dal = np.zeros(cl)
        for t in range(cl):
            v = Gam[t] * A[:, t] + Gp[t] * F[:, t]
            for j in range(t): v = v + beta(al, j, t - 1) * H[j, t] * K[:, j]
            for m in range(t + 1, cl): v = v - beta(al, t, m - 1) * st[m] * J[m, t] * K[:, m]
            dkg[:, t] = -st[t] * v
            ddl[:, t] = -st[t] * A[:, t]
            dst[t] = -J[t, t]
            a = Gam[t] * Gp[t] * trD
            for m in range(t + 1, cl): a -= Gam[t] * beta(al, t, m - 1) * st[m] * L[m]
            for j in range(t): a += Gp[t] * beta(al, j, t - 1) * ud[j]
            for j in range(t):
                for m in range(t + 1, cl):
                    a -= beta(al, j, t - 1) * beta(al, t, m - 1) * st[m] * H[j, m] * Gm[j, m]
            dal[t] = a
        DY = dys[s0:s1].T
        dQt = S0[:d].T @ DY; dQ = P.T @ dQt; Qt = P @ Q
        dProj = np.zeros_like(Proj)
        for t in range(cl):
            p = torch.tensor(Proj[:, t], requires_grad=True)
            k, dl, s, a, q = gates_t(p, d, eta_scale, alpha_bias, eps, eta_map)
            lo = (k * torch.tensor(dkg[:, t])).sum() + (dl * torch.tensor(ddl[:, t])).sum() + s * dst[t] + a * dal[t] + (q * torch.tensor(dQ[:, t])).sum()
            lo.backward(); dProj[:, t] = p.grad.numpy()
        dXt = S0[d:].T @ dProj
        dxs[s0:s1] = (P.T @ dXt).T
        bC = np.array([beta(al, j, cl - 1) for j in range(cl)])
        dS0[:d] += DY @ Qt.T
        dS0[d:] += dProj @ Xt.T
        dP = np.prod(al) * dP + Z @ np.diag(bC) @ U.T + dXt @ X.T + dQt @ Q.T
    dS0 += 0
    # the initial state adjoint: S_b = S0 P_c: all terms already in S0 coordinates
    return dxs, dS0

def scan_bwd(x, init, nh, g, chunk=0, **kw):
    B, H, W, D = x.shape; d = D // nh; N = H * W
    gx = np.zeros_like(x); gi = np.zeros_like(init)
    for b in range(B):
        for h in range(nh):
            for r in range(4):
                order = route_order(H, W, r)
                xs = x[b].reshape(N, D)[order, h*d:(h+1)*d]
                dys = g[b].reshape(N, D)[order, h*d:(h+1)*d]
                S0 = init[r, h].reshape(4*d + 2, d)
                dxs, dS0 = chain(xs, S0, dys, route_chunk(H, W, r, chunk), **kw)
                tmp = np.zeros((N, d)); tmp[order] = dxs
                gx[b].reshape(N, D)[:, h*d:(h+1)*d] += tmp
                gi[r, h] += dS0.reshape(-1)
    return gx, gi



CASES = {
    "aligned": (1, 3, 4, 8, 2, 0, dict(eta_scale=2.0)),
    "chunk5_softplus": (2, 4, 3, 4, 1, 5, dict(eta_map="softplus", eta_scale=0.5, alpha_bias=1.0)),
    "clamps": (1, 3, 3, 6, 1, 2, dict(eta_scale=40.0, alpha_bias=-1.0)),
    "longer": (1, 5, 6, 16, 1, 0, dict(eta_scale=3.0)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_chunk_parallel_backward_equals_gradient_oracle(name):
    B, H, W, D, nh, chunk, kw = CASES[name]
    rng = np.random.Generator(np.random.PCG64(1))
    d = D // nh
    S = 4 * d * d + 2 * d
    x = rng.standard_normal((B, H, W, D))
    init = rng.standard_normal((4, nh, S)) / np.sqrt(d)
    g = rng.standard_normal((B, H, W, D))
    gx, gi = scan_bwd(x, init, nh, g, chunk, **kw)
    rx, ri = hb.scan2d_backward(x, init, nh, g, chunk=chunk, **kw)
    assert np.abs(gx - rx).max() <= 1e-12 * np.abs(rx).max()
    assert np.abs(gi - ri).max() <= 1e-12 * np.abs(ri).max()


# The blocked form of the d = 32 kernel (backward_wy32.hip): each chunk is cut into blocks of
# TB tokens; G_s, the gain before a block, replaces I in the low-rank forms, the adjoint of
# each block's end gain is carried to the previous block, and P_c's adjoint picks up
# dP_{c+1} G_C^T with G_C the chunk's end gain.
# With the running readout y_t = S0[mem] P_c G_{t-1} q_t, the readout adjoint r_t = P_c^T S0[mem]^T dy_t
# enters every earlier gain: dG_{t-1} gains r_t q_t^T, so inside a block
#   dG_t = Gam'_t dG_e + sum_{m>t} beta_{t,m-1} (r_m q_m^T - step_m a_m k_m^T),
# the a-recurrence's base gains sum_{m>t} beta_{t,m-1} (q_m . k_t) r_m, dk and dalpha gain the
# matching terms, dq_t = G_{t-1}^T r_t, and the readout's reads of P_c and S0[mem] use
# G_{t-1} q_t in place of q_t.
def chain_blocked(xs, S0, dys, C, TB, eta_scale=1.0, alpha_bias=4.0, eps=1e-6, eta_map="sigmoid",
                  readout="boundary"):
    N, d = xs.shape
    nck = (N + C - 1) // C
    I = np.eye(d)
    running = readout == "running"

    def beta(al, j, t):  # prod_{i=j+1..t} al_i
        return float(np.prod(al[j + 1:t + 1]))

    def block_fwd(P, Gs, s0, s1):
        X = xs[s0:s1].T
        Xt = P @ X
        Proj = S0[d:] @ Xt
        c = s1 - s0
        K = np.zeros((d, c)); Dl = np.zeros((d, c)); Q = np.zeros((d, c)); st = np.zeros(c); al = np.zeros(c)
        for t in range(c):
            k, dl, s, a, q = gates_t(torch.tensor(Proj[:, t]), d, eta_scale, alpha_bias, eps, eta_map)
            K[:, t], Dl[:, t], Q[:, t], st[t], al[t] = k.numpy(), dl.numpy(), q.numpy(), float(s), float(a)
        Gm = K.T @ K
        Gk = Gs @ K
        U = np.zeros((d, c)); Wm = np.zeros((d, c))
        for t in range(c):
            acc = float(np.prod(al[:t])) * Gk[:, t] + Dl[:, t]
            for j in range(t):
                acc = acc + beta(al, j, t - 1) * Gm[j, t] * U[:, j]
            Wm[:, t] = acc
            U[:, t] = -st[t] * acc
        bE = np.array([beta(al, j, c - 1) for j in range(c)])
        Ge = np.prod(al) * Gs + U @ np.diag(bE) @ K.T
        # G_{t-1} q_t: what the running readout reads (q_t itself for the boundary readout)
        RQ = Q.copy()
        if running:
            for t in range(c):
                acc = float(np.prod(al[:t])) * (Gs @ Q[:, t])
                for j in range(t):
                    acc = acc + beta(al, j, t - 1) * float(K[:, j] @ Q[:, t]) * U[:, j]
                RQ[:, t] = acc
        return X, Xt, Proj, K, Dl, Q, st, al, Gm, Gk, U, Wm, Ge, RQ

    def blocks(c):
        s0, s1 = c * C, min(N, (c + 1) * C)
        return [(b0, min(s1, b0 + TB)) for b0 in range(s0, s1, TB)]

    # forward sweep: P_c and every block's start gain
    P = I.copy(); Ps = []; starts = []
    for c in range(nck):
        Ps.append(P.copy())
        Gs = I.copy(); st_c = []
        for b0, b1 in blocks(c):
            st_c.append(Gs.copy())
            Gs = block_fwd(P, Gs, b0, b1)[-2]
        starts.append((st_c, Gs))
        P = P @ Gs
    dPn = np.zeros((d, d)); dS0 = np.zeros_like(S0); dxs = np.zeros_like(xs)
    for c in range(nck - 1, -1, -1):
        P = Ps[c]
        st_c, GC = starts[c]
        dG = P.T @ dPn
        dPc = dPn @ GC.T
        for i in range(len(st_c) - 1, -1, -1):
            b0, b1 = blocks(c)[i]
            Gs = st_c[i]
            X, Xt, Proj, K, Dl, Q, st, al, Gm, Gk, U, Wm, _, RQ = block_fwd(P, Gs, b0, b1)
            cl = b1 - b0
            Gam = np.array([np.prod(al[:t]) for t in range(cl)])        # Gamma_{t-1}
            Gp = np.array([np.prod(al[t + 1:]) for t in range(cl)])     # Gamma'_t
            E = dG @ K; F = dG.T @ Wm; trD = np.sum(Gs * dG); ud = np.sum(U * E, 0)
            DY = dys[b0:b1].T
            dQt = S0[:d].T @ DY
            R = P.T @ dQt                                                # readout adjoints r_t
            A = np.zeros((d, cl))
            for t in range(cl - 1, -1, -1):
                acc = Gp[t] * E[:, t]
                for m in range(t + 1, cl):
                    acc = acc - beta(al, t, m - 1) * st[m] * Gm[m, t] * A[:, m]
                    if running:
                        acc = acc + beta(al, t, m - 1) * float(Q[:, m] @ K[:, t]) * R[:, m]
                A[:, t] = acc
            H = U.T @ A; J = A.T @ Wm; L = np.sum(Gk * A, 0); GA = Gs.T @ A
            dkg = np.zeros((d, cl)); ddl = np.zeros((d, cl)); dst = np.zeros(cl); dal = np.zeros(cl)
            dQ = R.copy()                                                # G_{t-1}^T r_t (running)
            for t in range(cl):
                v = Gam[t] * GA[:, t] + Gp[t] * F[:, t]
                for j in range(t): v = v + beta(al, j, t - 1) * H[j, t] * K[:, j]
                for m in range(t + 1, cl): v = v - beta(al, t, m - 1) * st[m] * J[m, t] * K[:, m]
                if running:
                    for m in range(t + 1, cl): v = v + beta(al, t, m - 1) * float(R[:, m] @ Wm[:, t]) * Q[:, m]
                dkg[:, t] = -st[t] * v
                ddl[:, t] = -st[t] * A[:, t]
                dst[t] = -J[t, t]
                a = Gam[t] * Gp[t] * trD
                for m in range(t + 1, cl): a -= Gam[t] * beta(al, t, m - 1) * st[m] * L[m]
                for j in range(t): a += Gp[t] * beta(al, j, t - 1) * ud[j]
                for j in range(t):
                    for m in range(t + 1, cl):
                        a -= beta(al, j, t - 1) * beta(al, t, m - 1) * st[m] * H[j, m] * Gm[j, m]
                if running:
                    for m in range(t + 1, cl):
                        a += Gam[t] * beta(al, t, m - 1) * float(R[:, m] @ (Gs @ Q[:, m]))
                        for j in range(t):
                            a += (beta(al, j, t - 1) * beta(al, t, m - 1) * float(U[:, j] @ R[:, m])
                                  * float(K[:, j] @ Q[:, m]))
                    dQ[:, t] = Gam[t] * (Gs.T @ R[:, t])
                    for j in range(t): dQ[:, t] += beta(al, j, t - 1) * float(U[:, j] @ R[:, t]) * K[:, j]
                dal[t] = a
            Qt = P @ RQ
            dProj = np.zeros_like(Proj)
            for t in range(cl):
                p = torch.tensor(Proj[:, t], requires_grad=True)
                k, dl, s, a, q = gates_t(p, d, eta_scale, alpha_bias, eps, eta_map)
                lo = (k * torch.tensor(dkg[:, t])).sum() + (dl * torch.tensor(ddl[:, t])).sum() + s * dst[t] + a * dal[t] + (q * torch.tensor(dQ[:, t])).sum()
                lo.backward(); dProj[:, t] = p.grad.numpy()
            dXt = S0[d:].T @ dProj
            dxs[b0:b1] = (P.T @ dXt).T
            dS0[:d] += DY @ Qt.T
            dS0[d:] += dProj @ Xt.T
            dPc += dXt @ X.T + dQt @ RQ.T
            dG = np.prod(al) * dG - (A * (Gam * st)) @ K.T
            if running:
                dG = dG + (R * Gam) @ Q.T
        dPn = dPc
    return dxs, dS0


def scan_bwd_blocked(x, init, nh, g, chunk, TB, **kw):
    B, H, W, D = x.shape; d = D // nh; N = H * W
    gx = np.zeros_like(x); gi = np.zeros_like(init)
    for b in range(B):
        for h in range(nh):
            for r in range(4):
                order = route_order(H, W, r)
                xs = x[b].reshape(N, D)[order, h*d:(h+1)*d]
                dys = g[b].reshape(N, D)[order, h*d:(h+1)*d]
                S0 = init[r, h].reshape(4*d + 2, d)
                dxs, dS0 = chain_blocked(xs, S0, dys, route_chunk(H, W, r, chunk), TB, **kw)
                tmp = np.zeros((N, d)); tmp[order] = dxs
                gx[b].reshape(N, D)[:, h*d:(h+1)*d] += tmp
                gi[r, h] += dS0.reshape(-1)
    return gx, gi


#            B, H, W, D, nh, chunk, TB, options
BLOCKED_CASES = {
    "rows7_blocks3": (1, 3, 7, 6, 1, 0, 3, dict(eta_scale=2.0)),           # 7-token rows: blocks 3, 3, 1
    "chunk10_blocks4_softplus": (1, 4, 5, 8, 2, 10, 4, dict(eta_map="softplus", eta_scale=0.5, alpha_bias=1.0)),
    "clamps_blocks2": (1, 3, 4, 6, 1, 5, 2, dict(eta_scale=40.0, alpha_bias=-1.0)),
    "chunk20_blocks16": (1, 4, 10, 4, 1, 20, 16, dict(eta_scale=3.0)),      # one full and one 4-token block
    "running_rows7_blocks3": (1, 3, 7, 6, 1, 0, 3, dict(eta_scale=2.0, readout="running")),
    "running_chunk10_blocks4_softplus": (1, 4, 5, 8, 2, 10, 4, dict(eta_map="softplus", eta_scale=0.5,
                                                                  alpha_bias=1.0, readout="running")),
    "running_clamps_blocks2": (1, 3, 4, 6, 1, 5, 2, dict(eta_scale=40.0, alpha_bias=-1.0, readout="running")),
}


@pytest.mark.parametrize("name", list(BLOCKED_CASES))
def test_blocked_backward_equals_gradient_oracle(name):
    B, H, W, D, nh, chunk, TB, kw = BLOCKED_CASES[name]
    rng = np.random.Generator(np.random.PCG64(2))
    d = D // nh
    S = 4 * d * d + 2 * d
    x = rng.standard_normal((B, H, W, D))
    init = rng.standard_normal((4, nh, S)) / np.sqrt(d)
    g = rng.standard_normal((B, H, W, D))
    gx, gi = scan_bwd_blocked(x, init, nh, g, chunk, TB, **kw)
    rx, ri = hb.scan2d_backward(x, init, nh, g, chunk=chunk, **kw)
    assert np.abs(gx - rx).max() <= 1e-12 * np.abs(rx).max()
    assert np.abs(gi - ri).max() <= 1e-12 * np.abs(ri).max()
