"""fp64 CPU oracle for the four-direction Hope memory scan.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  The product path (the
HIP library and its Python binding) never calls it, and it shares no code with
that path: the two meet only in the seeded inputs of ``workloads``.

The oracle is the method written out plainly, token by token, in float64,
following the pages' order and notation.  Sources (cited by page title and
section / equation):

  [VH]  "VisionHOPE: Visual Backbones as Self-Modifying Learning Systems"
  [NLz] "Nested Learning: the 'illusion' of deep learning architectures and
         multi-timescale memory" (Chinese reading notes on Nested Learning)
  [VM]  "VMamba: Visual State Space Model" (explainer page)
  [NL]  "Nested Learning: The Illusion of Deep Learning Architectures", part 12

What is computed, per image b, head h and selected route r:
  * the route order p_r(t) ([VM] "Four orders give each position several views
    of the image"; [VH] Sec. 2.3, Eq. 24);
  * chunks aligned with rows / columns ([VH] Sec. 2.3, Eq. 25);
  * per chunk, quantities generated from the memories frozen at the chunk start
    ([VH] Sec. 2.1.3, Eq. 15-16; [NLz] Sec. 2.10 on the chunk-start index);
  * the executed step of the stability-matched control ([VH] Sec. 2.2,
    Definition 1, Eq. 19-20, with the finite-precision safeguards of App. B.3);
  * the self-referential retained-DGD update of every memory, token by token
    ([VH] Sec. 2.1.2, Eq. 13, with the chunked signal of Eq. 16);
  * the readout y_t = M^m_b q_t and the restore-and-sum merge ([VH] Eq. 16 and
    Eq. 26 with unit scales; [VM] "Cross-merge restores positions before adding").

Readings where the pages leave a step open:
  * six memories: VisionHOPE's five plus the query memory M_q that the Nested
    Learning update set (Eq. 96) contains; q_t = n(M_q,b x_t) and every memory
    follows the same update;
  * q is normalised like k: q = q_raw / sqrt(|q_raw|^2 + 1e-6);
  * gate maps: eta = eta_scale * sigmoid(s) (default) or eta_scale * softplus(s)
    ([VH] App. C.1, Eq. 53); alpha = sigmoid(s + alpha_bias);
  * the inward factor (1 - 1e-3) multiplies eta_inj before the soft cap; the
    spectral limit is multiplied by (1 - 1e-6), its |k|^2 floored at 1e-20 and
    the result moved one ulp toward zero in the working precision;
  * eta_bar = 0 when eta = 0 or eta_inj = 0 (the cap's 0/0 limit).
"""
from __future__ import annotations

import numpy as np

MEMORIES = ("mem", "k", "v", "q", "eta", "alpha")
ROUTES = (0, 1, 2, 3)            # ->, <-, down, up
INJ_INWARD = 1.0 - 1e-3
SPEC_INWARD = 1.0 - 1e-6
KAPPA_FLOOR = 1e-20
NORM_EPS = 1e-6


# --------------------------------------------------------------------------
# Route orders: [VM] "Four orders give each position several views of the
# image" and [VH] Sec. 2.3 Eq. 24.  Row-major flattening, the flattening of the
# spatial transpose, and the full reversal of each.
# --------------------------------------------------------------------------
def route_order(H: int, W: int, r: int) -> np.ndarray:
    """p_r(t): flat pixel index (h * W + w) visited at sequence step t."""
    grid = np.arange(H * W, dtype=np.int64).reshape(H, W)
    if r == 0:
        return grid.reshape(-1)
    if r == 1:
        return grid.reshape(-1)[::-1].copy()
    if r == 2:
        return grid.T.reshape(-1)
    if r == 3:
        return grid.T.reshape(-1)[::-1].copy()
    raise ValueError("route index must be 0..3")


def route_chunk(H: int, W: int, r: int, chunk: int) -> int:
    """Chunk length of route r: [VH] Sec. 2.3 Eq. 25 when chunk == 0."""
    if chunk > 0:
        return chunk
    return W if r in (0, 1) else H


def cross_scan(x: np.ndarray, r: int) -> np.ndarray:
    """Serialise x[B, H, W, D] along route r -> [B, N, D]."""
    B, H, W, D = x.shape
    return x.reshape(B, H * W, D)[:, route_order(H, W, r), :]


def cross_merge(routes: dict, H: int, W: int) -> np.ndarray:
    """Restore each route's [B, N, D] output to the grid and add, per pixel,
    in the fixed order ->, <-, down, up ([VH] Eq. 26 with lambda_r = 1)."""
    first = next(iter(routes.values()))
    B, N, D = first.shape
    out = np.zeros((B, N, D), dtype=np.float64)
    for r in ROUTES:
        if r not in routes:
            continue
        order = route_order(H, W, r)
        y = routes[r]
        for t in range(N):
            out[:, order[t], :] += y[:, t, :]
    return out.reshape(B, H, W, D)


# --------------------------------------------------------------------------
# Gate maps: [VH] App. C.1 Eq. 53 (softplus form) and the sigmoid form of the
# synthetic workloads.
# --------------------------------------------------------------------------
def sigmoid(s):
    return 1.0 / (1.0 + np.exp(-s))


def phi_eta(s, eta_map: str = "sigmoid", eta_scale: float = 1.0):
    if eta_map == "sigmoid":
        return eta_scale * sigmoid(s)
    if eta_map == "softplus":
        return eta_scale * np.logaddexp(0.0, s)
    raise ValueError(eta_map)


def phi_alpha(s, alpha_bias: float = 4.0):
    return sigmoid(s + alpha_bias)


def stabilized_normalize(z: np.ndarray, eps: float = NORM_EPS) -> np.ndarray:
    """z / sqrt(|z|^2 + eps) along the last axis ([VH] App. C.1, key normalisation)."""
    return z / np.sqrt(np.sum(z * z, axis=-1, keepdims=True) + eps)


# --------------------------------------------------------------------------
# Stability-matched step-size control: [VH] Sec. 2.2 Definition 1, Eq. 19-20,
# and the finite-precision safeguards of App. B.3.
# --------------------------------------------------------------------------
def soft_injection_cap(eta, alpha, delta, eps: float = NORM_EPS, inward: float = INJ_INWARD):
    """Eq. 19: returns (eta_bar, eta_inj) for one token or a batch of tokens."""
    eta = np.asarray(eta, dtype=np.float64)
    alpha = np.asarray(alpha, dtype=np.float64)
    r = np.sqrt(np.sum(delta * delta, axis=-1) + eps * eps) + eps
    eta_inj = inward * (1.0 - alpha) / r
    ok = (eta != 0.0) & (eta_inj != 0.0)
    safe_inj = np.where(ok, eta_inj, 1.0)
    eta_bar = np.where(ok, safe_inj * -np.expm1(-eta / safe_inj), 0.0)
    return eta_bar, eta_inj


def spectral_limit(alpha, k, inward: float = SPEC_INWARD, floor: float = KAPPA_FLOOR,
                   dtype=np.float64):
    """Eq. 20 with the App. B.3 safeguards, rounded one ulp toward zero in ``dtype``."""
    kappa = np.maximum(np.sum(k * k, axis=-1), floor)
    lim = (inward * 2.0 * np.asarray(alpha, dtype=np.float64) / kappa).astype(dtype)
    return np.nextafter(lim, dtype(0)).astype(np.float64)


def executed_step(eta, alpha, k, delta, eps: float = NORM_EPS, injection: str = "soft",
                  spectral: str = "clamp", counts: dict | None = None):
    """eta_tilde = min(eta_bar, eta_spec) ([VH] Eq. 20), or one of the ablation controls of
    [VH] Sec. 3.5:

      injection = "soft"  the soft injection cap of Eq. 19 (default);
                  "hard"  a hard clamp at the same injection limit, min(eta, eta_inj);
                  "none"  no injection control, eta_bar = eta;
      spectral  = "clamp" min(eta_bar, eta_spec) (default);
                  "soft"  a smooth map to the same spectral limit, taken as the saturating
                          map of Eq. 19 with eta_spec in place of eta_inj:
                          eta_spec (1 - exp(-eta_bar / eta_spec));
                  "none"  no spectral control, eta_tilde = eta_bar.

    counts (optional) accumulates, over live tokens: "updates"; "inj", tokens whose raw eta
    exceeds the injection limit (where a hard clamp binds); "spec", tokens whose eta_bar
    exceeds the spectral limit (where the clamp binds); and "inj_near" / "spec_near",
    tokens within a relative counts["near_rel"] (set by the caller, default 1e-5) of
    either boundary.
    """
    eta = np.asarray(eta, dtype=np.float64)
    eta_soft, eta_inj = soft_injection_cap(eta, alpha, delta, eps)
    if injection == "soft":
        eta_bar = eta_soft
    elif injection == "hard":
        eta_bar = np.minimum(eta, eta_inj)
    elif injection == "none":
        eta_bar = eta
    else:
        raise ValueError(injection)
    lim = spectral_limit(alpha, k)
    if spectral == "clamp":
        step = np.minimum(eta_bar, lim)
    elif spectral == "soft":
        ok = (eta_bar != 0.0) & (lim != 0.0)
        safe = np.where(ok, lim, 1.0)
        step = np.where(ok, safe * -np.expm1(-eta_bar / safe), 0.0)
    elif spectral == "none":
        step = eta_bar
    else:
        raise ValueError(spectral)
    if counts is not None:
        counts["updates"] = counts.get("updates", 0) + int(eta.size)
        counts["inj"] = counts.get("inj", 0) + int(np.sum(eta > eta_inj))
        counts["spec"] = counts.get("spec", 0) + int(np.sum(eta_bar > lim))
        band = counts.get("near_rel", 1e-5)
        counts["inj_near"] = counts.get("inj_near", 0) + int(np.sum(np.abs(eta - eta_inj) <= band * np.abs(eta_inj)))
        counts["spec_near"] = counts.get("spec_near", 0) + int(np.sum(np.abs(eta_bar - lim) <= band * np.abs(lim)))
    return step


# --------------------------------------------------------------------------
# One retained-DGD write: [VH] Sec. 2.1.1 Eq. 7 / Sec. 2.1.2 Eq. 13.
#   M <- M (alpha I - eta k k^T) - eta g k^T
# M is [n, rows, d] (a 1 x d row memory has rows = 1); k is [n, d]; g is
# [n, rows]; alpha, eta are [n].
# --------------------------------------------------------------------------
def retained_dgd(M, k, g, eta, alpha, dgd: bool = True):
    """dgd=False is the DGD ablation of [VH] Sec. 3.5: the key-dependent correction
    -eta M k k^T is removed, M <- alpha M - eta g k^T, keeping the output-space signal,
    the retention factor and the step control."""
    n, d = k.shape
    eye = np.broadcast_to(np.eye(d), (n, d, d))
    A = alpha[:, None, None] * eye
    if dgd:
        A = A - eta[:, None, None] * (k[:, :, None] * k[:, None, :])
    return M @ A - eta[:, None, None] * (g[:, :, None] * k[:, None, :])


def _matvec(M, x):
    """[n, rows, d] @ [n, d] -> [n, rows]."""
    return (M @ x[:, :, None])[:, :, 0]


# --------------------------------------------------------------------------
# One SRNL chain (one head of one route, possibly many chains in a batch):
# [VH] Sec. 2.1.3 Eq. 15-16 for generation from the chunk-start state,
# Eq. 19-20 for the step, Eq. 13 for the token-order update of each memory.
# --------------------------------------------------------------------------
def srnl_chain(xs: np.ndarray, state: dict, chunk: int, eta_map: str = "sigmoid",
               eta_scale: float = 1.0, alpha_bias: float = 4.0, eps: float = NORM_EPS,
               control: bool = True, log: list | None = None, readout: str = "boundary",
               injection: str = "soft", spectral: str = "clamp", frozen=(), dgd: bool = True,
               counts: dict | None = None, qs: np.ndarray | None = None,
               mem_chunk: int | None = None, norm_log: list | None = None):
    """Run chains over ordered tokens.

    xs    : [n, N, d] tokens in route order
    state : dict name -> [n, rows, d] initial memories (rows = d, or 1 for eta/alpha)
    chunk : chunk length C >= 1
    control=False executes the raw step eta (the uncontrolled recurrence of
    [VH] Eq. 17), used only to show that the checks can fail.
    readout="boundary" reads y_t = M^m_b q_t with the memory frozen at the chunk
    start ([VH] Eq. 16); "running" reads y_t = M^m_{t-1} q_t, the memory as updated
    by the chunk's earlier tokens ([NL] Eq. 94, y_t = M_memory,t-1 q_t, applied inside
    the chunk; the projections still come from the chunk-start memories).  Both
    agree when every chunk is one token.
    injection / spectral select the step controls (see executed_step); frozen names the
    memories held fixed within the image ([VH] Sec. 3.5: without adaptive K/V, frozen =
    ("k", "v"); without adaptive dynamics, ("eta", "alpha")); dgd=False removes the
    key-dependent correction of the update (retained_dgd).
    qs [n, N, d] (optional): queries given from outside in route order, the fixed outer
    query projection of [VH] App. B.5 (and Eq. 14); q_t is then qs_t normalised within the
    head like the generated one, and M_q takes no part (it stays at its initial value).
    mem_chunk (optional) gives the working memory M_mem its own chunk length, the two
    chunk sizes of [NLz] Sec. 2.10: M_mem's boundary state (its readout in the boundary
    form and its self-generated targets) is refreshed at multiples of mem_chunk, the other
    five memories' (which generate k, v, q, eta, alpha) at multiples of chunk.  None or
    chunk: one chunk size.
    norm_log (optional list): after each chunk, {"end": e, m: ||M_m||_F per chain for every
    memory m} is appended (the per-chunk memory norms).
    Returns (ys [n, N, d], final state dict).
    """
    for m in frozen:
        if m not in MEMORIES:
            raise ValueError(f"unknown memory {m!r}")
    if readout not in ("boundary", "running"):
        raise ValueError("readout must be 'boundary' or 'running'")
    xs = np.asarray(xs, dtype=np.float64)
    n, N, d = xs.shape
    cm = chunk if mem_chunk is None else int(mem_chunk)
    if cm < 1:
        raise ValueError("mem_chunk must be >= 1")
    M = {m: np.array(state[m], dtype=np.float64, copy=True) for m in MEMORIES}
    ys = np.zeros((n, N, d), dtype=np.float64)
    Mb = {}                                               # boundary states M_b
    for s in range(0, N, chunk):
        for m in MEMORIES:
            if m != "mem":
                Mb[m] = M[m].copy()
        for t in range(s, min(s + chunk, N)):
            if t % cm == 0:                               # the working memory's own boundary
                Mb["mem"] = M["mem"].copy()
            x = xs[:, t, :]
            k = stabilized_normalize(_matvec(Mb["k"], x), eps)
            v = _matvec(Mb["v"], x)
            q = stabilized_normalize(_matvec(Mb["q"], x) if qs is None else qs[:, t, :], eps)
            eta = phi_eta(_matvec(Mb["eta"], x)[:, 0], eta_map, eta_scale)
            alpha = phi_alpha(_matvec(Mb["alpha"], x)[:, 0], alpha_bias)
            # y_t = M^m_b q_t (boundary) or M^m_{t-1} q_t (running: M is not yet
            # updated with token t here)
            ys[:, t, :] = _matvec(Mb["mem"] if readout == "boundary" else M["mem"], q)
            delta = k - v
            step = (executed_step(eta, alpha, k, delta, eps, injection, spectral, counts)
                    if control else eta)
            if log is not None:
                log.append({"t": t, "eta": eta, "alpha": alpha, "step": step, "k": k,
                            "delta": delta})
            for m in MEMORIES:
                if m in frozen or (m == "q" and qs is not None):
                    continue
                vhat = _matvec(Mb[m], v)                      # self-generated target, Eq. 16
                g = _matvec(Mb[m], k) - vhat                  # output-space signal, Eq. 16
                M[m] = retained_dgd(M[m], k, g, step, alpha, dgd)  # Eq. 13
        if norm_log is not None:
            entry = {"end": min(s + chunk, N)}
            for m in MEMORIES:
                entry[m] = np.sqrt(np.sum(M[m] ** 2, axis=(1, 2)))
            norm_log.append(entry)
    return ys, M


def scan2d(x: np.ndarray, init: np.ndarray, n_heads: int, dirs: int = 15, chunk: int = 0,
           eta_map: str = "sigmoid", eta_scale: float = 1.0, alpha_bias: float = 4.0,
           eps: float = NORM_EPS, init_per_image: bool = False, heads=None, images=None,
           readout: str = "boundary", injection: str = "soft", spectral: str = "clamp",
           frozen=(), dgd: bool = True, route_scales=None, skip=None,
           shared_init: bool = False, counts: dict | None = None, queries=None,
           mem_chunk: int = 0, step_map: np.ndarray | None = None):
    """The whole operator: serialise, run every (image, head, route) chain, merge.

    x    : [B, H, W, D] (any float dtype; widened to fp64)
    init : [4, n_heads, S] (or [B, 4, n_heads, S] with init_per_image), S = 4d^2 + 2d,
           per (route, head) the flat concatenation M_mem, M_k, M_v, M_q (row-major
           d x d), m_eta, m_alpha.
    heads / images restrict the computation to a subset (sampled checks); the
    returned arrays then cover only those.
    route_scales [4, D] are the channel-wise direction scales lambda_r of [VH] Eq. 26
    (None: unit scales); skip [D] is the channel-wise skip of [VH] App. B.5, added to each
    route's head-wise reads before its scale: Y_r = reads_r + skip * Z_r.
    shared_init: init is [n_heads, S], the same initial memories for every route (the
    shared-initial-state variant of [VH] Sec. 3.5; trajectories stay separate).
    readout, injection, spectral, frozen, dgd: see srnl_chain; counts accumulates the
    step-control counters of executed_step over every chain computed.
    queries [B, H, W, D] (optional): the fixed-projection queries of [VH] App. B.5, computed
    once per image and reused by every route (serialised like x, split into heads).
    mem_chunk > 0 gives the working memory its own chunk length (srnl_chain); 0 keeps one
    chunk size for all six memories.
    step_map [b, 4, h, H, W] (optional, filled in place): the executed step eta_tilde of
    [VH] Eq. 20 (or of the selected ablation control) of every token of a computed chain,
    at the token's pixel, indexed by route; entries of unselected routes are not written.
    The step maps are the per-pixel view of the step controls that [VH] Sec. 3.5 inspects.
    Returns (out [b, H, W, D_sel] fp64, final [b, 4, h, S] fp64, NaN for
    unselected routes).
    """
    x = np.asarray(x, dtype=np.float64)
    B, H, W, D = x.shape
    d = D // n_heads
    heads = list(range(n_heads)) if heads is None else list(heads)
    images = list(range(B)) if images is None else list(images)
    xb = x[images]
    nb = len(images)
    S = 4 * d * d + 2 * d
    init = np.asarray(init, dtype=np.float64)
    out = np.zeros((nb, H, W, len(heads) * d), dtype=np.float64)
    final = np.full((nb, 4, len(heads), S), np.nan, dtype=np.float64)
    for hi, h in enumerate(heads):
        routes = {}
        for r in ROUTES:
            if not (dirs >> r) & 1:
                continue
            xs = cross_scan(xb[..., h * d:(h + 1) * d], r)
            if shared_init:
                flat = np.broadcast_to(init[h], (nb, S))
            elif init_per_image:
                flat = init[images, r, h]
            else:
                flat = np.broadcast_to(init[r, h], (nb, S))
            st = unflatten_state(flat, d)
            C = route_chunk(H, W, r, chunk)
            qs = None
            if queries is not None:
                qsel = np.asarray(queries, dtype=np.float64)[images]
                qs = cross_scan(qsel[..., h * d:(h + 1) * d], r)
            log = [] if step_map is not None else None
            ys, fin = srnl_chain(xs, st, C, eta_map, eta_scale, alpha_bias, eps, readout=readout,
                                 injection=injection, spectral=spectral, frozen=frozen, dgd=dgd,
                                 counts=counts, qs=qs, mem_chunk=mem_chunk if mem_chunk > 0 else None,
                                 log=log)
            if log is not None:                       # token t of route r sits at pixel order[t]
                order = route_order(H, W, r)
                for entry in log:
                    pix = order[entry["t"]]
                    step_map[:, r, hi, pix // W, pix % W] = entry["step"]
            if skip is not None:                      # Y_r = reads + skip * Z_r  ([VH] App. B.5)
                ys = ys + np.asarray(skip, dtype=np.float64)[h * d:(h + 1) * d] * xs
            if route_scales is not None:              # lambda_r * Y_r  ([VH] Eq. 26)
                ys = ys * np.asarray(route_scales, dtype=np.float64)[r, h * d:(h + 1) * d]
            routes[r] = ys
            final[:, r, hi, :] = flatten_state(fin)
        if routes:
            out[..., hi * d:(hi + 1) * d] = cross_merge(routes, H, W)
    return out, final


def unflatten_state(flat: np.ndarray, d: int) -> dict:
    flat = np.asarray(flat, dtype=np.float64)
    dd = d * d
    st = {}
    for i, m in enumerate(("mem", "k", "v", "q")):
        st[m] = flat[..., i * dd:(i + 1) * dd].reshape(flat.shape[:-1] + (d, d)).copy()
    st["eta"] = flat[..., 4 * dd:4 * dd + d].reshape(flat.shape[:-1] + (1, d)).copy()
    st["alpha"] = flat[..., 4 * dd + d:].reshape(flat.shape[:-1] + (1, d)).copy()
    return st


def flatten_state(st: dict) -> np.ndarray:
    lead = st["k"].shape[:-2]
    parts = [st[m].reshape(lead + (-1,)) for m in MEMORIES]
    return np.concatenate(parts, axis=-1)


# --------------------------------------------------------------------------
# Second form of the same chunk: the shared right-multiplicative gain of
# [VH] App. B.4 Prop. 2, Eq. 46 (G_b = I, G_t = G_{t-1} A_t + B_t with
# A_t = alpha_t I - eta_t k k^T and B_t = -eta_t delta k^T, Eq. 21).
# Used by the tests to check the literal per-memory loop, not by scan2d.
# --------------------------------------------------------------------------
def chunk_gain(k, delta, step, alpha):
    """k, delta: [n, C, d]; step, alpha: [n, C] -> list of G_t, t = b..b+C ([n, d, d])."""
    n, C, d = k.shape
    G = np.broadcast_to(np.eye(d), (n, d, d)).copy()
    out = [G.copy()]
    for t in range(C):
        kt = k[:, t]
        A = alpha[:, t, None, None] * np.eye(d) - step[:, t, None, None] * (kt[:, :, None] * kt[:, None, :])
        Bm = -step[:, t, None, None] * (delta[:, t, :, None] * kt[:, None, :])
        G = G @ A + Bm
        out.append(G.copy())
    return out
