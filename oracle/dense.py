"""Dense fp64 oracle: explicit cost matrix, log-sum-exp half-steps, residual,
annealed solve, entropic row materializer and the ``min_row`` threshold.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Conventions (the readings are listed with their reasons in the design notes):
  * cost           C_ij = s * sum_k (x_ik - y_jk)^2, s a number resolved once
                   (moscot #846, "Two correctness traps": the scale is captured
                   as a resolved value, never re-derived from a subset);
  * plan           pi_ij = a_i b_j exp((f_i + g_j - C_ij) / eps)
                   (FlashSinkhorn 2, §2.1: entropic OT with an eps-weighted KL
                   term; moscot #846 "Fix": entropic rows exp((f+g-C)/eps) with
                   the weights carried by the plan);
  * f half-step    f_i = -eps * LSE_j( log b_j + (g_j - C_ij)/eps )
  * g half-step    g_j = -eps * LSE_i( log a_i + (f_i - C_ij)/eps )
                   (FlashSinkhorn 2, §2.1: log-domain Sinkhorn alternates the
                   source and target dual updates);
  * LSE over an all -inf row is -inf (POT #868, "Tests": the all -inf row);
  * residual       R_row = sum_i |sum_j pi_ij - a_i|, R_col likewise
                   (FlashSinkhorn 2, §3.1 and §A.1: L1 marginal residual).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_CHUNK_ELEMS = 1 << 22  # fp64 entries per explicit cost chunk (32 MiB)


def _f64(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float64)


def _threads() -> int:
    """Worker threads: ORACLE_THREADS, else OMP_NUM_THREADS, else the CPUs
    this process may run on (the thread count never changes a result: every
    chunk is computed alone and the chunks are combined in order)."""
    for var in ("ORACLE_THREADS", "OMP_NUM_THREADS"):
        env = os.environ.get(var, "").strip()
        if env.isdigit():
            return max(1, int(env))
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except (AttributeError, OSError):
        return max(1, os.cpu_count() or 1)


def _chunks(count: int, width: int):
    step = max(1, _CHUNK_ELEMS // max(1, width))
    return [(s, min(count, s + step)) for s in range(0, count, step)]


def _map_chunks(fn, count, width, threads=None):
    """Apply ``fn(lo, hi)`` to row chunks; numpy releases the GIL inside."""
    spans = _chunks(count, width)
    threads = _threads() if threads is None else threads
    if threads <= 1 or len(spans) == 1:
        return [fn(lo, hi) for lo, hi in spans]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(lambda s: fn(*s), spans))


def cost_rows(x, y, scale: float, rows=None) -> np.ndarray:
    """Explicit C[rows, :] = s * sum_k (x_ik - y_jk)^2 in float64.

    FlashSinkhorn 2, §2.1 (squared-Euclidean cost) with the scale resolved to
    a number as in moscot #846 ("Two correctness traps").
    """
    x = _f64(x)
    y = _f64(y)
    xr = x if rows is None else x[np.asarray(rows)]
    C = np.zeros((xr.shape[0], y.shape[0]))
    for k in range(x.shape[1]):
        diff = xr[:, k][:, None] - y[:, k][None, :]
        C += diff * diff
    return float(scale) * C


def logsumexp_rows(Z: np.ndarray) -> np.ndarray:
    """LSE over axis 1 with an explicit max shift; an all -inf row gives -inf."""
    Z = _f64(Z)
    M = Z.max(axis=1)
    out = np.full(Z.shape[0], -np.inf)
    ok = np.isfinite(M)
    if ok.any():
        shifted = Z[ok] - M[ok][:, None]
        out[ok] = M[ok] + np.log(np.exp(shifted).sum(axis=1))
    # a row holding +inf has LSE +inf
    out[M == np.inf] = np.inf
    return out


def _log_weights(w) -> np.ndarray:
    w = _f64(w)
    with np.errstate(divide="ignore"):
        return np.log(w)


def halfstep_f(x, y, b, g, eps: float, scale: float, rows=None, threads=None) -> np.ndarray:
    """f_i = -eps * LSE_j(log b_j + (g_j - C_ij)/eps) for i in ``rows`` (all if None).

    FlashSinkhorn 2, §2.1: the source dual update of log-domain Sinkhorn.
    """
    x = _f64(x)
    y = _f64(y)
    g = _f64(g)
    lb = _log_weights(b)
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    eps = float(eps)

    def run(lo, hi):
        C = cost_rows(x, y, scale, rows[lo:hi])
        Z = lb[None, :] + (g[None, :] - C) / eps
        return -eps * logsumexp_rows(Z)

    parts = _map_chunks(run, len(rows), y.shape[0], threads)
    return np.concatenate(parts) if parts else np.zeros(0)


def halfstep_g(x, y, a, f, eps: float, scale: float, cols=None, threads=None) -> np.ndarray:
    """g_j = -eps * LSE_i(log a_i + (f_i - C_ij)/eps): the target dual update
    (FlashSinkhorn 2, §2.1), i.e. the source update with the roles swapped."""
    return halfstep_f(y, x, a, f, eps, scale, rows=cols, threads=threads)


def plan_rows(x, y, a, b, f, g, eps: float, scale: float, rows=None) -> np.ndarray:
    """pi[rows, :] = a_i b_j exp((f_i + g_j - C_ij)/eps), formed explicitly."""
    rows = np.arange(len(x)) if rows is None else np.asarray(rows)
    C = cost_rows(x, y, scale, rows)
    E = (_f64(f)[rows][:, None] + _f64(g)[None, :] - C) / float(eps)
    return _f64(a)[rows][:, None] * _f64(b)[None, :] * np.exp(E)


def marginal_residuals(x, y, a, b, f, g, eps: float, scale: float, threads=None):
    """(R_row, R_col) = (sum_i |sum_j pi_ij - a_i|, sum_j |sum_i pi_ij - b_j|).

    The plan is formed explicitly chunk by chunk (FlashSinkhorn 2, §3.1: the
    exact residual is an O(nm) pass; §A.1: the L1 row residual).
    """
    n = len(x)
    m = len(y)

    def run(lo, hi):
        P = plan_rows(x, y, a, b, f, g, eps, scale, np.arange(lo, hi))
        return P.sum(axis=1), P.sum(axis=0)

    parts = _map_chunks(run, n, m, threads)
    row_sums = np.concatenate([p[0] for p in parts])
    col_sums = np.zeros(m)
    for p in parts:
        col_sums += p[1]
    R_row = float(np.abs(row_sums - _f64(a)).sum())
    R_col = float(np.abs(col_sums - _f64(b)).sum())
    return R_row, R_col


def row_residual_identity(a, f, f_next, eps: float) -> float:
    """sum_i a_i |exp((f_i - f~_i)/eps) - 1|, f~ the f half-step at the same g.

    Right after an f half-step every row of the plan sums to a_i, so the row
    sums at (f, g) are a_i exp((f_i - f~_i)/eps); this is R_row without
    forming the plan.
    """
    d = (_f64(f) - _f64(f_next)) / float(eps)
    return float((_f64(a) * np.abs(np.exp(d) - 1.0)).sum())


def mean_sqeuclid(x, y) -> float:
    """Unweighted mean of ||x_i - y_j||^2 over all n*m pairs, by explicit sum.

    This is the ``scale_cost="mean"`` statistic that moscot #846 resolves once
    over the full clouds ("Two correctness traps").
    """
    x = _f64(x)
    y = _f64(y)

    def run(lo, hi):
        return cost_rows(x, y, 1.0, np.arange(lo, hi)).sum()

    total = math.fsum(_map_chunks(run, len(x), len(y)))
    return total / (len(x) * len(y))


@dataclass
class Schedule:
    """Annealing schedule (FlashSinkhorn 2, §3.1 and §B.2: the coarse stage
    anneals; Table 2 context: continuation in eps).

    Stages eps_start, eps_start*eps_factor, ... while above eps_target, each
    running ``iters_per_stage`` full iterations (warm started). Then eps_target:
    exactly ``fixed_iters`` iterations if that is positive, else iterate until
    max(R_row, R_col) <= tol, at most ``max_iters`` iterations.
    """

    eps_start: float
    eps_target: float
    eps_factor: float = 0.5
    iters_per_stage: int = 10
    fixed_iters: int = 0
    tol: float = 1e-3
    max_iters: int = 10000


def annealing_stages(s: Schedule) -> list[float]:
    """The eps values strictly above eps_target, by repeated multiplication."""
    out = []
    eps = float(s.eps_start)
    while eps > s.eps_target:
        out.append(eps)
        eps = eps * float(s.eps_factor)
    return out


@dataclass
class SolveResult:
    f: np.ndarray
    g: np.ndarray
    iters: int  # full iterations in total (annealing + final stage)
    final_iters: int  # full iterations at eps_target
    R_row: float
    R_col: float
    converged: bool
    history: list = field(default_factory=list)


def solve(x, y, a, b, scale: float, sched: Schedule, f0=None, g0=None, threads=None) -> SolveResult:
    """Annealed log-domain Sinkhorn: f then g per iteration, f = g = 0 start.

    FlashSinkhorn 2, §2.1 (alternating updates) and §3.1 (annealing); the
    stop test max(R_row, R_col) <= tol is applied after every full iteration
    at eps_target only.
    """
    f = np.zeros(len(x)) if f0 is None else _f64(f0).copy()
    g = np.zeros(len(y)) if g0 is None else _f64(g0).copy()
    iters = 0
    for eps in annealing_stages(sched):
        for _ in range(sched.iters_per_stage):
            f = halfstep_f(x, y, b, g, eps, scale, threads=threads)
            g = halfstep_g(x, y, a, f, eps, scale, threads=threads)
            iters += 1
    eps = float(sched.eps_target)
    history = []
    final = 0
    converged = False
    R = (math.nan, math.nan)
    if sched.fixed_iters > 0:
        for _ in range(sched.fixed_iters):
            f = halfstep_f(x, y, b, g, eps, scale, threads=threads)
            g = halfstep_g(x, y, a, f, eps, scale, threads=threads)
            iters += 1
            final += 1
        R = marginal_residuals(x, y, a, b, f, g, eps, scale, threads=threads)
        history.append(R)
        converged = True
    else:
        while final < sched.max_iters:
            f = halfstep_f(x, y, b, g, eps, scale, threads=threads)
            g = halfstep_g(x, y, a, f, eps, scale, threads=threads)
            iters += 1
            final += 1
            R = marginal_residuals(x, y, a, b, f, g, eps, scale, threads=threads)
            history.append(R)
            if max(R) <= sched.tol:
                converged = True
                break
    return SolveResult(f, g, iters, final, R[0], R[1], converged, history)


def materialize_rows(x, y, a, b, f, g, eps: float, scale: float, rows) -> np.ndarray:
    """T[rows, :] = a_i b_j exp((f_i + g_j - C_ij)/eps) (moscot #846, "Fix",
    entropic outputs), computed row by row from the explicit cost."""
    return plan_rows(x, y, a, b, f, g, eps, scale, rows)


def min_row(x, y, a, b, f, g, eps: float, scale: float) -> float:
    """min over rows with a_i > 0 of max_j T_ij (moscot #846, "Behavioural
    changes": the largest threshold that keeps every row; massless rows take
    no part in choosing it)."""
    x = _f64(x)
    live = np.nonzero(_f64(a) > 0)[0]
    if live.size == 0:
        return math.nan

    def run(lo, hi):
        return plan_rows(x, y, a, b, f, g, eps, scale, live[lo:hi]).max(axis=1)

    return float(np.concatenate(_map_chunks(run, live.size, len(y))).min())


def sparsify(x, y, a, b, f, g, eps: float, scale: float, threshold: float):
    """The plan entries >= threshold as CSR (row_ptr int64, col int64, val
    float64), rows in order and columns increasing within a row.

    moscot pull request #846: rows are thresholded from the materialized plan
    rows, so only the surviving values and indices are kept; a threshold > 0
    leaves rows without mass empty.
    """
    ptr = [0]
    cols, vals = [], []
    for lo, hi in _chunks(len(x), len(y)):
        T = plan_rows(x, y, a, b, f, g, eps, scale, rows=np.arange(lo, hi))
        for r in range(T.shape[0]):
            keep = np.nonzero(T[r] >= threshold)[0]
            cols.append(keep)
            vals.append(T[r, keep])
            ptr.append(ptr[-1] + len(keep))
    col = np.concatenate(cols) if cols else np.zeros(0, np.int64)
    val = np.concatenate(vals) if vals else np.zeros(0)
    return np.asarray(ptr, np.int64), col.astype(np.int64), val
