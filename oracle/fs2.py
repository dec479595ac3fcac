"""Multiscale pipeline: Morton cells, coarse annealed Sinkhorn on cell records,
lift to points, and the sparse fine loop with a certified stop.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FlashSinkhorn 2:
  * §3 and §B.1: cells are Morton-prefix groups, at most twice as many cells
    as blocks; read here as the prefix of p = floor(log2(2 * max(NB, MB))) bits.
  * §3.1 and §B.2: the coarse stage anneals on cell records (centroid, mass),
    then lifts the potentials to points; extra centroid updates run until the
    coarse error stalls or 2048 updates.
  * §1, §A.1: the lift of centroid potentials to the points is a log-sum-exp
    against the other side's centroids (worked example: two points at -h, h
    per side in one cell give lifted residual cosh(2h^2/eps) - 1).
  * §3.2: every fine update rebuilds the mask at the current potentials and
    runs both sparse half-steps on it.
  * §3.2 (with §C.5): optionally, the screened tiles are verified with their
    exact row and column shares before the half-steps (``verify_tiles``), and
    both supports come from the survivors.
  * §3.1 and §B.2 (optional adaptive switch): the coarse stage runs in batches
    of centroid updates; after each, the lifted potentials are accepted when
    est + 3 SE < tol on both sides, est and SE being the sampled estimate of
    the L1 marginal residual and its standard error (1024 sampled indices per
    side, expanded to 8192 when that
    interval straddles tol, the same samples at every check); otherwise more
    centroid updates follow until they stall or reach their cap, and the fine
    loop takes over. Sample indices: the raw outputs of Philox4x64-10 keyed
    (seed, side) (numpy's ``Philox``), each reduced modulo the side's size.
  * §C.4: the stop certificate is the admitted-plan residual plus a bound on
    the omitted mass. Read here as R_A + Omega <= tol with
    Omega = max(NB, MB) * delta_rel, the a-priori total omitted-mass bound
    of the threshold rule (§3.2).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .blocks import (
    block_summaries,
    compact_tiles,
    screen,
    screen_transpose,
    sparse_halfstep_f,
    sparse_halfstep_g,
    sparse_residuals,
    verify_tiles,
)
from .dense import Schedule, annealing_stages, halfstep_f, halfstep_g, marginal_residuals, plan_rows
from .morton import BITS, morton_order


def cells(codes_sorted, P_sorted, w_sorted, p_bits: int):
    """Cells = runs of equal Morton prefix (top ``p_bits`` bits of the d*21-bit
    code). Returns offsets int64 [C+1], centroids [C,d] = sum w x / sum w
    (plain mean for a massless cell) and masses [C] = sum w, in float64."""
    codes = np.asarray(codes_sorted, dtype=np.uint64)
    P = np.asarray(P_sorted, dtype=np.float64)
    w = np.asarray(w_sorted, dtype=np.float64)
    d = P.shape[1]
    shift = np.uint64(d * BITS - p_bits)
    prefix = codes >> shift
    starts = np.concatenate([[0], np.nonzero(prefix[1:] != prefix[:-1])[0] + 1])
    offsets = np.concatenate([starts, [len(codes)]]).astype(np.int64)
    C = len(starts)
    cent = np.empty((C, d))
    mass = np.empty(C)
    for c in range(C):
        s, e = offsets[c], offsets[c + 1]
        ws = w[s:e]
        mass[c] = ws.sum()
        if mass[c] > 0:
            cent[c] = (ws[:, None] * P[s:e]).sum(axis=0) / mass[c]
        else:
            cent[c] = P[s:e].mean(axis=0)
    return offsets, cent, mass


def lift(P, cent_q, mass_q, G, eps: float, scale: float) -> np.ndarray:
    """Point potentials from the other side's centroid potentials:
    f_i = -eps * LSE_J(log M_J + (G_J - s ||p_i - c_J||^2)/eps)."""
    return halfstep_f(P, cent_q, mass_q, G, eps, scale)


@dataclass
class FS2Params:
    B: int = 128
    eps: float = 1e-4
    tol: float = 1e-2
    delta_scale: float = 1e-3  # delta_rel = delta_scale / max(NB, MB)
    coarse_eps_start: float = 1.0
    coarse_factor: float = 0.5
    coarse_iters_per_stage: int = 10
    coarse_tol: float = 1e-3
    coarse_max: int = 2048
    stall_window: int = 10
    stall_rel: float = 0.01
    max_fine: int = 8192
    p_bits: int = -1  # -1: floor(log2(2 * max(NB, MB)))
    scale: float = 1.0
    verify: bool = False  # exact share check of the screened tiles
    adaptive: bool = False  # sampled lift checks between batches of coarse updates
    check_every: int = 128  # coarse updates per batch
    check_samples: int = 1024
    check_samples_max: int = 8192
    sample_seed: int = 0


@dataclass
class FS2Result:
    f: np.ndarray  # user order
    g: np.ndarray
    coarse_iters: int
    fine_updates: int
    R_A_row: float
    R_A_col: float
    omega: float
    certified: bool
    ncells_x: int
    ncells_y: int
    tiles_history: list = field(default_factory=list)
    candidates_history: list = field(default_factory=list)
    accepted_by_sample: bool = False
    checks: int = 0
    check_history: list = field(default_factory=list)  # (R_row, SE_row, R_col, SE_col, samples)


def prefix_bits(NB: int, MB: int, d: int) -> int:
    """Morton prefix length of a cell (§3, §B.1: at most twice as many cells
    as blocks): the largest p with 2^p <= 2 * max(NB, MB), at most the code
    length d * 21, so no side has more than 2 * max(NB, MB) cells."""
    return min(d * BITS, int(math.floor(math.log2(2 * max(NB, MB)))))


def coarse_solve(cx, cy, mx, my, prm: FS2Params):
    """Annealed dense Sinkhorn between centroid clouds, then iterations at the
    target eps until R <= coarse_tol, a stall, or coarse_max updates."""
    F = np.zeros(len(cx))
    G = np.zeros(len(cy))
    iters = 0
    sched = Schedule(prm.coarse_eps_start, prm.eps, prm.coarse_factor, prm.coarse_iters_per_stage)
    for eps in annealing_stages(sched):
        for _ in range(prm.coarse_iters_per_stage):
            F = halfstep_f(cx, cy, my, G, eps, prm.scale)
            G = halfstep_g(cx, cy, mx, F, eps, prm.scale)
            iters += 1
    hist = []
    for _ in range(prm.coarse_max):
        F = halfstep_f(cx, cy, my, G, prm.eps, prm.scale)
        G = halfstep_g(cx, cy, mx, F, prm.eps, prm.scale)
        iters += 1
        hist.append(max(marginal_residuals(cx, cy, mx, my, F, G, prm.eps, prm.scale)))
        if coarse_done(hist, prm):
            break
    return F, G, iters


def coarse_done(hist, prm: FS2Params) -> bool:
    """Stop rule of the centroid updates at the target eps, given the residual
    history R_1..R_k of those updates (§3.1, §B.2: extra centroid updates run
    until the coarse error stalls; the cap of 2048 updates is the caller's
    loop bound). Read here as: stop once R_k <= coarse_tol, or once the last
    ``stall_window`` updates cut the residual by less than the fraction
    ``stall_rel``, i.e. R_k > (1 - stall_rel) * R_{k - stall_window}."""
    R = hist[-1]
    if R <= prm.coarse_tol:
        return True
    w = prm.stall_window
    return len(hist) > w and R > (1.0 - prm.stall_rel) * hist[-1 - w]


def sample_indices(count: int, k: int, seed: int, stream: int) -> np.ndarray:
    """k indices in [0, count), uniform with replacement: the first k raw
    outputs of Philox4x64-10 keyed (seed, stream), each modulo count."""
    raw = np.random.Philox(key=np.array([seed, stream], dtype=np.uint64)).random_raw(k)
    return (raw % np.uint64(count)).astype(np.int64)


def sampled_residual(P, Q, wp, wq, fp, gq, eps: float, scale: float, idx):
    """(estimate, standard error) of R = sum_i |sum_j pi_ij - a_i| from the
    rows idx drawn uniformly with replacement: count * mean(t) and
    count * std(t, ddof=1) / sqrt(k), t = |sum_j pi_ij - a_i| of each drawn row
    (FlashSinkhorn 2, §3.1: sampled row sums cost O(md))."""
    rows = np.asarray(idx, np.int64)
    T = plan_rows(P, Q, wp, wq, fp, gq, eps, scale, rows=rows)
    t = np.abs(T.sum(axis=1) - np.asarray(wp, np.float64)[rows])
    k = len(rows)
    est = len(P) * float(t.mean())
    se = len(P) * float(t.std(ddof=1)) / math.sqrt(k) if k > 1 else math.inf
    return est, se


def lift_accepted(X, Y, A, Bw, f, g, prm):
    """The sampled check of lifted potentials: (accepted, (R_row, SE_row,
    R_col, SE_col, samples))."""
    k = prm.check_samples
    while True:
        er, sr = sampled_residual(X, Y, A, Bw, f, g, prm.eps, prm.scale,
                                  sample_indices(len(X), k, prm.sample_seed, 0))
        ec, sc = sampled_residual(Y, X, Bw, A, g, f, prm.eps, prm.scale,
                                  sample_indices(len(Y), k, prm.sample_seed, 1))
        info = (er, sr, ec, sc, k)
        hi = max(er + 3.0 * sr, ec + 3.0 * sc)
        lo = max(er - 3.0 * sr, ec - 3.0 * sc)
        if hi < prm.tol:
            return True, info
        if lo >= prm.tol or k >= prm.check_samples_max:
            return False, info
        k = prm.check_samples_max


def coarse_batch(cx, cy, mx, my, F, G, prm, count: int, anneal: bool):
    """Optionally the annealing stages, then up to ``count`` updates at the
    target eps, stopping early when R <= coarse_tol or the residual stalls
    (stall window counted within the batch). Returns F, G, the annealing
    updates, the updates at the target eps, and done (converged or stalled)."""
    iters = 0
    annealed = 0
    if anneal:
        sched = Schedule(prm.coarse_eps_start, prm.eps, prm.coarse_factor, prm.coarse_iters_per_stage)
        for eps in annealing_stages(sched):
            for _ in range(prm.coarse_iters_per_stage):
                F = halfstep_f(cx, cy, my, G, eps, prm.scale)
                G = halfstep_g(cx, cy, mx, F, eps, prm.scale)
                annealed += 1
    hist = []
    for _ in range(count):
        F = halfstep_f(cx, cy, my, G, prm.eps, prm.scale)
        G = halfstep_g(cx, cy, mx, F, prm.eps, prm.scale)
        iters += 1
        hist.append(max(marginal_residuals(cx, cy, mx, my, F, G, prm.eps, prm.scale)))
        if coarse_done(hist, prm):
            return F, G, annealed, iters, True
    return F, G, annealed, iters, False


def fs2_solve(x, y, a, b, prm: FS2Params) -> FS2Result:
    x = np.asarray(x, np.float32)
    y = np.asarray(y, np.float32)
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    n, d = x.shape
    m = len(y)
    B = prm.B
    NB, MB = (n + B - 1) // B, (m + B - 1) // B
    delta = prm.delta_scale / max(NB, MB)
    omega = max(NB, MB) * delta
    p_bits = prm.p_bits if prm.p_bits > 0 else prefix_bits(NB, MB, d)

    cxs, px, cys, py = morton_order(x, y)
    X, Y, A, Bw = x[px], y[py], a[px], b[py]
    offx, centx, massx = cells(cxs, X, A, p_bits)
    offy, centy, massy = cells(cys, Y, Bw, p_bits)

    accepted = False
    checks = []
    if prm.adaptive:
        F = np.zeros(len(centx))
        G = np.zeros(len(centy))
        coarse_iters = 0
        at_eps = 0
        while True:
            count = min(prm.check_every, prm.coarse_max - at_eps)
            F, G, ann, it, done = coarse_batch(centx, centy, massx, massy, F, G, prm, count,
                                               coarse_iters == 0)
            at_eps += it
            coarse_iters += ann + it
            f = lift(X, centy, massy, G, prm.eps, prm.scale)
            g = lift(Y, centx, massx, F, prm.eps, prm.scale)
            accepted, info = lift_accepted(X, Y, A, Bw, f.astype(np.float32), g.astype(np.float32), prm)
            checks.append(info)
            if accepted or done or at_eps >= prm.coarse_max:
                break
    else:
        F, G, coarse_iters = coarse_solve(centx, centy, massx, massy, prm)
        f = lift(X, centy, massy, G, prm.eps, prm.scale)
        g = lift(Y, centx, massx, F, prm.eps, prm.scale)
    if accepted:
        fu = np.empty(n)
        gu = np.empty(m)
        fu[px] = f
        gu[py] = g
        return FS2Result(fu, gu, coarse_iters, 0, math.nan, math.nan, omega, False,
                         len(centx), len(centy), [], [], True, len(checks), checks)

    tiles = []
    cands = []
    certified = False
    R_row = R_col = math.nan
    updates = 0
    while True:
        f32 = f.astype(np.float32)
        g32 = g.astype(np.float32)
        sx = block_summaries(X, A, f32, B)
        sy = block_summaries(Y, Bw, g32, B)
        ptr, col = screen(sx, sy, prm.eps, prm.scale, delta)
        cands.append(int(ptr[-1]))
        if prm.verify:
            keep = verify_tiles(X, Y, A, Bw, f32, g32, prm.eps, prm.scale, ptr, col, B, delta)
            ptr, col, ptrT, rowT = compact_tiles(ptr, col, keep, len(sy[2]))
        else:
            ptrT, rowT = screen_transpose(sx, sy, prm.eps, prm.scale, delta)
        tiles.append(int(ptr[-1]))
        R_row, R_col = sparse_residuals(X, Y, A, Bw, f, g, prm.eps, prm.scale, ptr, col, ptrT, rowT, B)
        if max(R_row, R_col) + omega <= prm.tol:
            certified = True
            break
        if updates >= prm.max_fine:  # R_row, R_col belong to the returned state
            break
        f = sparse_halfstep_f(X, Y, Bw, g, prm.eps, prm.scale, ptr, col, B)
        g = sparse_halfstep_g(X, Y, A, f, prm.eps, prm.scale, ptrT, rowT, B)
        updates += 1

    fu = np.empty(n)
    gu = np.empty(m)
    fu[px] = f
    gu[py] = g
    return FS2Result(fu, gu, coarse_iters, updates, R_row, R_col, omega, certified,
                     len(centx), len(centy), tiles, cands, False, len(checks), checks)
