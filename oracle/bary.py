"""Barycentric projection of plan rows and the source-coordinate gradient.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FlashSinkhorn 2: Block-Sparse Entropic Optimal Transport:
  * §A.2: holding the target side and its potentials fixed, the gradient of
    the objective with respect to source point z_i is 2 a_i (z_i - T_i), with
    T_i the barycentric projection of row i of the plan, i.e. the mean of the
    targets under the row's conditional weights. With the cost scale s of
    C_ij = s ||x_i - y_j||^2 the same derivation gives 2 s a_i (x_i - T_i).
  * §A.4: the masked (sparse) gradient takes the projection over the admitted
    tiles only.

The conditional weights of row i are pi_ij / sum_j pi_ij; with
pi_ij = a_i b_j exp((f_i + g_j - C_ij)/eps) the row factor a_i exp(f_i/eps)
cancels, so T_i depends on g only: w_ij proportional to b_j exp((g_j - C_ij)/eps).
"""
from __future__ import annotations

import numpy as np

from .blocks import _nblocks, _support
from .dense import cost_rows


def _project(xr, Q, lb, g, eps, scale):
    """Rows of T for source rows xr against targets Q (log-weights lb)."""
    C = cost_rows(xr, Q, scale)
    Z = lb[None, :] + (g[None, :] - C) / float(eps)
    M = Z.max(axis=1)
    W = np.exp(Z - M[:, None])
    return (W @ np.asarray(Q, np.float64)) / W.sum(axis=1)[:, None]


def _log_weights(w):
    w = np.asarray(w, np.float64)
    return np.log(w, where=w > 0, out=np.full(len(w), -np.inf))


def barycentric_rows(x, y, b, g, eps: float, scale: float, rows=None) -> np.ndarray:
    """T[rows] = sum_j w_ij y_j / sum_j w_ij, w_ij = b_j exp((g_j - C_ij)/eps)."""
    x = np.asarray(x, np.float64)
    rows = np.arange(len(x)) if rows is None else np.asarray(rows)
    return _project(x[rows], y, _log_weights(b), np.asarray(g, np.float64), eps, scale)


def coordinate_gradient(x, a, T, scale: float) -> np.ndarray:
    """grad_i = 2 s a_i (x_i - T_i)  (FlashSinkhorn 2, §A.2)."""
    x = np.asarray(x, np.float64)
    a = np.asarray(a, np.float64)
    return 2.0 * float(scale) * a[:, None] * (x - np.asarray(T, np.float64))


def sparse_barycentric_rows(P, Q, wq, g, eps: float, scale: float, ptr, col, B: int) -> np.ndarray:
    """The projection restricted to each row block's admitted tiles (all
    columns for a block with none), as in the masked gradient (§A.4)."""
    P = np.asarray(P, np.float64)
    lb = _log_weights(wq)
    g = np.asarray(g, np.float64)
    n, m = len(P), len(Q)
    T = np.empty((n, P.shape[1]))
    for I in range(_nblocks(n, B)):
        s, e = I * B, min(n, (I + 1) * B)
        js = _support(ptr, col, I, B, m)
        T[s:e] = _project(P[s:e], np.asarray(Q)[js], lb[js], g[js], eps, scale)
    return T
