"""Pins for the block screen and sparse half-steps: brute-force omitted-mass
bounds (FlashSinkhorn 2, §A.3), shift invariance, transposition, and the
reduction to the dense update when every tile is admitted."""
import math

import numpy as np
import pytest
from scipy.spatial.distance import cdist

import oracle


def _clustered(rng, n, m):
    cx = rng.uniform(0, 1, size=(6, 3))
    x = cx[rng.integers(0, 6, n)] + rng.normal(0, 0.03, size=(n, 3))
    y = cx[rng.integers(0, 6, m)] + rng.normal(0, 0.03, size=(m, 3)) + 0.02
    x = x.astype(np.float32)
    y = y.astype(np.float32)
    a = rng.uniform(0.5, 1.5, n)
    b = rng.uniform(0.5, 1.5, m)
    a = (a / a.sum()).astype(np.float32)
    b = (b / b.sum()).astype(np.float32)
    _, px, _, py = oracle.morton_order(x, y)
    return x[px], y[py], a[px], b[py]


def _potentials(x, y, a, b, eps, iters=30):
    res = oracle.solve(x, y, a, b, 1.0, oracle.Schedule(0.5, eps, iters_per_stage=3, fixed_iters=iters))
    return res.f.astype(np.float32), res.g.astype(np.float32)


@pytest.fixture(scope="module")
def problem():
    rng = np.random.default_rng(7)
    x, y, a, b = _clustered(rng, 640, 560)
    eps = 2e-3
    f, g = _potentials(x, y, a, b, eps)
    return x, y, a, b, f, g, eps


def _dense_mask(ptr, col, NB, MB):
    M = np.zeros((NB, MB), bool)
    for I in range(NB):
        M[I, col[ptr[I]:ptr[I + 1]]] = True
    return M


def test_omitted_tiles_respect_row_and_column_bounds(problem):
    x, y, a, b, f, g, eps = problem
    B = 32
    NB, MB = math.ceil(len(x) / B), math.ceil(len(y) / B)
    delta = 1e-3 / max(NB, MB)
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, delta)
    M = _dense_mask(ptr, col, NB, MB)
    assert 0 < M.sum() < NB * MB  # neither empty nor dense
    C = cdist(x.astype(np.float64), y.astype(np.float64), "sqeuclidean")
    P = (a.astype(np.float64)[:, None] * b.astype(np.float64)[None, :]
         * np.exp((f.astype(np.float64)[:, None] + g.astype(np.float64)[None, :] - C) / eps))
    for I in range(NB):
        for J in range(MB):
            if M[I, J]:
                continue
            tile = P[I * B:(I + 1) * B, J * B:(J + 1) * B]
            assert np.all(tile.sum(1) <= delta * a[I * B:(I + 1) * B] * (1 + 1e-12))
            assert np.all(tile.sum(0) <= delta * b[J * B:(J + 1) * B] * (1 + 1e-12))
    # total omitted mass on either side is at most max(NB, MB) * delta
    omitted = P * ~np.kron(M, np.ones((B, B), bool))[:len(x), :len(y)]
    assert omitted.sum(1).sum() <= MB * delta and omitted.sum(0).sum() <= NB * delta


def test_screen_shift_invariance_and_transpose(problem):
    x, y, a, b, f, g, eps = problem
    B = 32
    delta = 1e-4
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, delta)
    k = np.float32(0.25)
    sx2 = oracle.block_summaries(x, a, f + k, B)
    sy2 = oracle.block_summaries(y, b, g - k, B)
    ptr2, col2 = oracle.screen(sx2, sy2, eps, 1.0, delta)
    assert np.array_equal(ptr, ptr2) and np.array_equal(col, col2)
    ptrT, rowT = oracle.screen_transpose(sx, sy, eps, 1.0, delta)
    NB, MB = len(ptr) - 1, len(ptrT) - 1
    assert np.array_equal(_dense_mask(ptr, col, NB, MB).T, _dense_mask(ptrT, rowT, MB, NB))


def test_sparse_equals_dense_when_all_tiles_admitted(problem):
    x, y, a, b, f, g, eps = problem
    B = 64
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, 1e-300)
    assert ptr[-1] == len(sx[2]) * len(sy[2])
    fs = oracle.sparse_halfstep_f(x, y, b, g, eps, 1.0, ptr, col, B)
    np.testing.assert_allclose(fs, oracle.halfstep_f(x, y, b, g, eps, 1.0), rtol=1e-13, atol=1e-15)


def test_sparse_equals_masked_lse(problem):
    x, y, a, b, f, g, eps = problem
    B = 32
    NB, MB = math.ceil(len(x) / B), math.ceil(len(y) / B)
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, 1e-2 / NB)
    M = np.kron(_dense_mask(ptr, col, NB, MB), np.ones((B, B), bool))[:len(x), :len(y)]
    empty = ~M.any(1)
    M[empty] = True  # a row block with no admitted tile takes the dense update
    C = cdist(x.astype(np.float64), y.astype(np.float64), "sqeuclidean")
    Z = np.where(M, np.log(b.astype(np.float64))[None, :] + (g.astype(np.float64)[None, :] - C) / eps, -np.inf)
    from scipy.special import logsumexp

    expected = -eps * logsumexp(Z, axis=1)
    fs = oracle.sparse_halfstep_f(x, y, b, g, eps, 1.0, ptr, col, B)
    np.testing.assert_allclose(fs, expected, rtol=1e-12, atol=1e-15)


def test_sparse_residual_plus_omega_bounds_full_residual(problem):
    x, y, a, b, f, g, eps = problem
    B = 32
    NB, MB = math.ceil(len(x) / B), math.ceil(len(y) / B)
    delta = 1e-3 / max(NB, MB)
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, delta)
    ptrT, rowT = oracle.screen_transpose(sx, sy, eps, 1.0, delta)
    Rr, Rc = oracle.sparse_residuals(x, y, a, b, f, g, eps, 1.0, ptr, col, ptrT, rowT, B)
    Fr, Fc = oracle.marginal_residuals(x, y, a, b, f, g, eps, 1.0)
    omega = max(NB, MB) * delta
    assert Fr <= Rr + omega + 1e-12 and Fc <= Rc + omega + 1e-12


def test_single_point_blocks_reduce_to_the_plan_threshold(rng):
    """With B = 1 every bound is tight: F = f, G = g, D = C and W = weight, so a
    pair is omitted iff pi_ij <= delta * min(a_i, b_j)."""
    n, m = 40, 30
    x = rng.uniform(0, 1, size=(n, 3)).astype(np.float32)
    y = rng.uniform(0, 1, size=(m, 3)).astype(np.float32)
    a = rng.pareto(1.5, n) + 0.05
    b = rng.pareto(1.5, m) + 0.05
    a = (a / a.sum()).astype(np.float32)
    b = (b / b.sum()).astype(np.float32)
    eps = 0.02
    g = np.zeros(m)
    f = oracle.halfstep_f(x, y, b, g, eps, 1.0).astype(np.float32)
    g = oracle.halfstep_g(x, y, a, f, eps, 1.0).astype(np.float32)
    P = oracle.plan_rows(x, y, a, b, f.astype(np.float64), g.astype(np.float64), eps, 1.0)
    thr = np.minimum(a.astype(np.float64)[:, None], b.astype(np.float64)[None, :])
    for delta in (1e-3, 1e-2, 0.1):
        keep = P > delta * thr
        ratio = P / (delta * thr)
        assert np.all(np.abs(ratio - 1) > 1e-9)  # no pair sits on the boundary
        ptr, col = oracle.screen(oracle.block_summaries(x, a, f, 1), oracle.block_summaries(y, b, g, 1),
                                 eps, 1.0, delta)
        assert np.array_equal(_dense_mask(ptr, col, n, m), keep)
        assert 0 < keep.sum() < n * m


def test_row_block_without_admitted_tiles_takes_the_dense_update(problem):
    x, y, a, b, f, g, eps = problem
    B = 32
    f = f.copy()
    f[:B] -= np.float32(1.0)  # rows of block 0 carry almost no mass
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, 1e-3 / len(sx[2]))
    assert ptr[1] == ptr[0]
    fs = oracle.sparse_halfstep_f(x, y, b, g, eps, 1.0, ptr, col, B)
    dense = oracle.halfstep_f(x[:B], y, b, g, eps, 1.0)
    np.testing.assert_allclose(fs[:B], dense, rtol=1e-13)
