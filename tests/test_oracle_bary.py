"""Pins of the barycentric projection and coordinate gradient oracle
(FlashSinkhorn 2, §A.2 and §A.4) against closed forms, limits and a finite
difference of the entropic OT value."""
import numpy as np
import pytest

import oracle
from oracle.dense import Schedule


def _clouds(rng, n, m, d):
    x = rng.uniform(0, 1, size=(n, d))
    y = rng.uniform(0, 1, size=(m, d))
    a = rng.uniform(0.5, 1.5, n)
    b = rng.uniform(0.5, 1.5, m)
    return x, y, a / a.sum(), b / b.sum()


def test_identical_targets_project_onto_that_target(rng):
    x, y, a, b = _clouds(rng, 7, 5, 3)
    y[:] = y[2]
    g = rng.normal(0, 0.1, 5)
    T = oracle.barycentric_rows(x, y, b, g, 0.05, 1.0)
    np.testing.assert_allclose(T, np.broadcast_to(y[2], T.shape), rtol=0, atol=1e-15)


def test_large_eps_gives_the_weighted_target_mean(rng):
    x, y, a, b = _clouds(rng, 6, 9, 2)
    T = oracle.barycentric_rows(x, y, b, np.zeros(9), 1e7, 1.0)
    mean = (b[:, None] * y).sum(0) / b.sum()
    np.testing.assert_allclose(T, np.broadcast_to(mean, T.shape), rtol=0, atol=1e-6)


def test_small_eps_picks_the_best_target(rng):
    x, y, a, b = _clouds(rng, 12, 10, 3)
    g = rng.normal(0, 0.05, 10)
    eps = 1e-6
    C = ((x[:, None, :] - y[None, :, :]) ** 2).sum(-1)
    best = np.argmin(C - g[None, :], axis=1)
    gap = np.sort(C - g[None, :], axis=1)
    assert np.all(gap[:, 1] - gap[:, 0] > 1e3 * eps)  # unique winners by a wide margin
    T = oracle.barycentric_rows(x, y, b, g, eps, 1.0)
    np.testing.assert_allclose(T, y[best], rtol=0, atol=1e-12)


def test_common_shift_of_g_leaves_the_projection(rng):
    x, y, a, b = _clouds(rng, 8, 11, 2)
    g = rng.normal(0, 0.1, 11)
    T0 = oracle.barycentric_rows(x, y, b, g, 0.02, 1.0)
    T1 = oracle.barycentric_rows(x, y, b, g + 3.7, 0.02, 1.0)
    np.testing.assert_allclose(T0, T1, rtol=0, atol=1e-13)


@pytest.mark.parametrize("scale", [1.0, 2.5])
def test_gradient_is_the_derivative_of_the_entropic_cost(rng, scale):
    """At convergence the entropic cost V(x) = <a, f> + <b, g> (primal = dual)
    has dV/dx_i = 2 s a_i (x_i - T_i): checked by central differences, each
    perturbed problem solved again to 1e-13."""
    x, y, a, b = _clouds(rng, 4, 5, 2)
    eps = 0.1
    sched = Schedule(eps, eps, tol=1e-13, max_iters=100000)

    def value(xx):
        r = oracle.solve(xx, y, a, b, scale, sched)
        assert r.converged
        return float(a @ r.f + b @ r.g), r

    _, r = value(x)
    T = oracle.barycentric_rows(x, y, b, r.g, eps, scale)
    G = oracle.coordinate_gradient(x, a, T, scale)
    h = 1e-5
    for i, k in [(0, 0), (1, 1), (3, 0), (2, 1)]:
        xp, xm = x.copy(), x.copy()
        xp[i, k] += h
        xm[i, k] -= h
        fd = (value(xp)[0] - value(xm)[0]) / (2 * h)
        assert fd == pytest.approx(G[i, k], rel=1e-6, abs=1e-10), (i, k, fd, G[i, k])


def test_sparse_projection_full_and_restricted_masks(rng):
    x, y, a, b = _clouds(rng, 10, 12, 2)
    g = rng.normal(0, 0.1, 12)
    B, eps = 4, 0.05
    NB, MB = 3, 3
    # every tile admitted: the dense projection
    ptr = np.arange(0, NB * MB + 1, MB)
    col = np.tile(np.arange(MB), NB)
    T = oracle.sparse_barycentric_rows(x, y, b, g, eps, 1.0, ptr, col, B)
    np.testing.assert_allclose(T, oracle.barycentric_rows(x, y, b, g, eps, 1.0), rtol=0, atol=1e-14)
    # row block 0 keeps column block 2 only; block 1 keeps 0 and 1; block 2 none (dense)
    ptr = np.array([0, 1, 3, 3])
    col = np.array([2, 0, 1])
    T = oracle.sparse_barycentric_rows(x, y, b, g, eps, 1.0, ptr, col, B)
    np.testing.assert_allclose(T[0:4], oracle.barycentric_rows(x[0:4], y[8:12], b[8:12], g[8:12], eps, 1.0),
                               rtol=0, atol=1e-14)
    np.testing.assert_allclose(T[4:8], oracle.barycentric_rows(x[4:8], y[0:8], b[0:8], g[0:8], eps, 1.0),
                               rtol=0, atol=1e-14)
    np.testing.assert_allclose(T[8:10], oracle.barycentric_rows(x[8:10], y, b, g, eps, 1.0), rtol=0, atol=1e-14)
