"""Block summaries, the block-pair screen, and sparse half-steps on its mask.

TEST INFRASTRUCTURE ONLY (see the package docstring).

All functions work on clouds already in Morton order (``oracle.morton``):
block I holds the consecutive points [I*B, min(n, (I+1)*B)).

FlashSinkhorn 2, §3.2 and §B.3: fine updates screen block pairs with
block-level potential maxima and bounding boxes, store admitted tiles in CSR
form, use a dense update for a block with no admitted tile, and run both
sparse half-steps on the same mask. §A.3: a tile whose upper bound is at most
its threshold omits at most delta_rel * a_i per row and delta_rel * b_j per
column, and the screen is invariant to (f + k, g - k).

Screen test, as read from those sections (the formulas are not printed):
for i in I and j in J, f_i <= F_I = max f, g_j <= G_J = max g and
C_ij >= D_IJ = s * sum_k max(0, lo_Jk - hi_Ik, lo_Ik - hi_Jk)^2, so
pi_ij <= a_i b_j u_IJ with u_IJ = exp((F_I + G_J - D_IJ)/eps). The omitted row
share of tile (I, J) is then at most a_i W_J u_IJ and the column share at most
b_j W_I u_IJ, with W = (points in block) * (largest weight in block). The tile
is omitted iff u_IJ * max(W_I, W_J) <= delta_rel, evaluated in float64 as

    (F_I + G_J) - D_IJ  <=  eps * (log(delta_rel) - max(log W_I, log W_J)),

with D_IJ accumulated axis by axis without fused multiply-adds and each
log taken by the C library's ``log`` (``math.log``) on the host.

Tile verification (§3.2: the screened candidates are checked with their exact
mass over the B^2 point pairs; §C.5 measures it). Read here as the exact form
of the same per-tile guarantee: with the row share of tile (I, J) for i in I
    s_i = sum_{j in J} b_j exp((f_i + g_j - C_ij)/eps)   (= sum_j pi_ij / a_i)
and the column share for j in J
    t_j = sum_{i in I} a_i exp((f_i + g_j - C_ij)/eps)   (= sum_i pi_ij / b_j),
a candidate is omitted iff every s_i <= delta_rel and every t_j <= delta_rel,
so each omitted tile still takes at most delta_rel * a_i from row i and
delta_rel * b_j from column j and the a-priori bound on the omitted mass is
unchanged. A block that would lose every candidate keeps them all (rows
first, then columns), so verification never turns a sparse block into a
dense one; keeping tiles never weakens the bound.
"""
from __future__ import annotations

import math

import numpy as np

from .dense import cost_rows, logsumexp_rows


def _nblocks(k: int, B: int) -> int:
    return (k + B - 1) // B


def block_summaries(P, w, pot, B: int):
    """Per block: lo [NB,d], hi [NB,d], Fmax [NB] (float64 of float32 values)
    and logW [NB] = log(count * max weight) by ``math.log``."""
    P = np.asarray(P, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32)
    pot = np.asarray(pot, dtype=np.float32)
    n, d = P.shape
    NB = _nblocks(n, B)
    lo = np.empty((NB, d))
    hi = np.empty((NB, d))
    F = np.empty(NB)
    logW = np.empty(NB)
    for I in range(NB):
        s, e = I * B, min(n, (I + 1) * B)
        lo[I] = P[s:e].min(axis=0)
        hi[I] = P[s:e].max(axis=0)
        F[I] = float(pot[s:e].max())
        W = float(e - s) * float(w[s:e].max())
        logW[I] = math.log(W) if W > 0 else -math.inf
    return lo, hi, F, logW


def _tile_keep(sx, sy, I, eps, scale, log_delta):
    """Boolean admit flags of row block I against every column block J."""
    lo_x, hi_x, F, lwx = sx
    lo_y, hi_y, G, lwy = sy
    d = lo_x.shape[1]
    acc = None
    for k in range(d):
        gap = np.maximum(np.maximum(lo_y[:, k] - hi_x[I, k], lo_x[I, k] - hi_y[:, k]), 0.0)
        sq = gap * gap
        acc = sq if acc is None else acc + sq
    D = float(scale) * acc
    lhs = (F[I] + G) - D
    rhs = float(eps) * (log_delta - np.maximum(lwx[I], lwy))
    return lhs > rhs


def screen(sx, sy, eps: float, scale: float, delta_rel: float, row_blocks=None):
    """Row-major CSR (row_ptr int64 [len+1], cols int32) of admitted tiles.

    ``sx``/``sy`` are ``block_summaries`` outputs of the source and target
    sides. ``row_blocks`` restricts the rows (all row blocks if None).
    """
    NB = sx[0].shape[0]
    rows = range(NB) if row_blocks is None else row_blocks
    log_delta = math.log(delta_rel)
    ptr = [0]
    cols = []
    for I in rows:
        keep = np.nonzero(_tile_keep(sx, sy, I, eps, scale, log_delta))[0]
        cols.append(keep.astype(np.int32))
        ptr.append(ptr[-1] + keep.size)
    col = np.concatenate(cols) if cols else np.zeros(0, np.int32)
    return np.asarray(ptr, dtype=np.int64), col.astype(np.int32)


def screen_transpose(sx, sy, eps: float, scale: float, delta_rel: float):
    """Column-major list of the same tiles: for each J, the admitted I in order.

    The test is symmetric in the two sides, so screening with the roles of the
    summaries swapped gives the transposed support.
    """
    return screen(sy, sx, eps, scale, delta_rel)


def _support(ptr, col, I, B, m):
    """Column indices of row block I: its admitted tiles, or all if none."""
    lo, hi = int(ptr[I]), int(ptr[I + 1])
    if hi == lo:
        return np.arange(m)
    parts = [np.arange(J * B, min(m, (J + 1) * B)) for J in col[lo:hi]]
    return np.concatenate(parts)


def sparse_halfstep_f(P, Q, wq, g, eps, scale, ptr, col, B):
    """f_i = -eps * LSE over the admitted columns of block(i) (dense if none).

    FlashSinkhorn 2, §3.2: CSR-streamed log-sum-exp over admitted tiles only;
    a block with no admitted tile takes a dense update.
    """
    n, m = len(P), len(Q)
    lb = np.log(np.asarray(wq, np.float64), where=np.asarray(wq) > 0,
                out=np.full(m, -np.inf))
    g = np.asarray(g, np.float64)
    f = np.empty(n)
    for I in range(_nblocks(n, B)):
        s, e = I * B, min(n, (I + 1) * B)
        js = _support(ptr, col, I, B, m)
        C = cost_rows(np.asarray(P)[s:e], np.asarray(Q)[js], scale)
        Z = lb[js][None, :] + (g[js][None, :] - C) / float(eps)
        f[s:e] = -float(eps) * logsumexp_rows(Z)
    return f


def sparse_halfstep_g(P, Q, wp, f, eps, scale, ptrT, rowsT, B):
    """g_j = -eps * LSE over the admitted rows of block(j), using the
    column-major support (FlashSinkhorn 2, §3.2: the transposed support)."""
    return sparse_halfstep_f(Q, P, wp, f, eps, scale, ptrT, rowsT, B)


def sparse_residuals(P, Q, wp, wq, f, g, eps, scale, ptr, col, ptrT, rowsT, B):
    """(R_A,row, R_A,col): L1 marginal residuals of the plan restricted to the
    supports (admitted tiles; all columns/rows for a block with none)."""
    P = np.asarray(P)
    Q = np.asarray(Q)
    wp = np.asarray(wp, np.float64)
    wq = np.asarray(wq, np.float64)
    f = np.asarray(f, np.float64)
    g = np.asarray(g, np.float64)
    n, m = len(P), len(Q)

    def side(P, Q, wp, wq, f, g, ptr, col):
        R = 0.0
        for I in range(_nblocks(len(P), B)):
            s, e = I * B, min(len(P), (I + 1) * B)
            js = _support(ptr, col, I, B, len(Q))
            C = cost_rows(P[s:e], Q[js], scale)
            pi = wp[s:e, None] * wq[None, js] * np.exp((f[s:e, None] + g[None, js] - C) / float(eps))
            R += float(np.abs(pi.sum(axis=1) - wp[s:e]).sum())
        return R

    return side(P, Q, wp, wq, f, g, ptr, col), side(Q, P, wq, wp, g, f, ptrT, rowsT)


def tile_shares(P, Q, wp, wq, f, g, eps: float, scale: float, I: int, J: int, B: int):
    """(s [rows of I], t [columns of J]): the row and column shares of tile
    (I, J) defined in the module docstring, in float64."""
    P = np.asarray(P)
    Q = np.asarray(Q)
    rs, re_ = I * B, min(len(P), (I + 1) * B)
    cs, ce = J * B, min(len(Q), (J + 1) * B)
    C = cost_rows(P[rs:re_], Q[cs:ce], scale)
    E = np.exp((np.asarray(f, np.float64)[rs:re_, None] + np.asarray(g, np.float64)[None, cs:ce] - C)
               / float(eps))
    s = E @ np.asarray(wq, np.float64)[cs:ce]
    t = np.asarray(wp, np.float64)[rs:re_] @ E
    return s, t


def verify_tiles(P, Q, wp, wq, f, g, eps: float, scale: float, ptr, col, B: int,
                 delta_rel: float):
    """Keep flags (bool per candidate, in CSR order) of the candidates (ptr,
    col) at potentials (f, g): a candidate stays unless every row share and
    every column share is <= delta_rel; then a row block that kept none of
    its candidates keeps them all, and after that a column block that kept
    none of its candidates keeps them all."""
    ptr = np.asarray(ptr, np.int64)
    col = np.asarray(col, np.int64)
    keep = np.zeros(len(col), dtype=bool)
    for I in range(len(ptr) - 1):
        for e in range(int(ptr[I]), int(ptr[I + 1])):
            s, t = tile_shares(P, Q, wp, wq, f, g, eps, scale, I, int(col[e]), B)
            keep[e] = bool((s > delta_rel).any() or (t > delta_rel).any())
    for I in range(len(ptr) - 1):
        lo, hi = int(ptr[I]), int(ptr[I + 1])
        if hi > lo and not keep[lo:hi].any():
            keep[lo:hi] = True
    for J in np.unique(col):
        sel = col == J
        if not keep[sel].any():
            keep[sel] = True
    return keep


def compact_tiles(ptr, col, keep, ncol_blocks: int):
    """The kept candidates as a row-major CSR (ptr, col) and the same tiles
    column-major (ptrT, rowsT: for each J the row blocks in increasing order)."""
    ptr = np.asarray(ptr, np.int64)
    col = np.asarray(col, np.int32)
    keep = np.asarray(keep, bool)
    nrow = len(ptr) - 1
    rows = np.repeat(np.arange(nrow, dtype=np.int32), np.diff(ptr))
    counts = np.array([int(keep[int(ptr[I]):int(ptr[I + 1])].sum()) for I in range(nrow)], np.int64)
    ptrV = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    colV = col[keep].astype(np.int32)
    rk = rows[keep]
    ptrT = [0]
    rowsT = []
    for J in range(ncol_blocks):
        r = rk[colV == J]
        rowsT.append(r)
        ptrT.append(ptrT[-1] + len(r))
    rowsT = np.concatenate(rowsT).astype(np.int32) if rowsT else np.zeros(0, np.int32)
    return ptrV, colV, np.asarray(ptrT, np.int64), rowsT
