"""Pins for the dense fp64 oracle, independent of the oracle's own code paths.

Each test checks the oracle against something the pages or the mathematics
fix: brute-force exp-domain Sinkhorn (scaling vectors u, v with a kernel built
by scipy), closed forms, invariants and special cases.
"""
import math

import numpy as np
import pytest
from scipy.spatial.distance import cdist

import oracle
from oracle import Schedule


def _clouds(rng, n, m, d):
    x = rng.uniform(0, 1, size=(n, d)).astype(np.float32)
    y = rng.normal(0.5, 0.2, size=(m, d)).astype(np.float32)
    a = rng.uniform(0.2, 1.0, size=n)
    b = rng.uniform(0.2, 1.0, size=m)
    a = (a / a.sum()).astype(np.float32)
    b = (b / b.sum()).astype(np.float32)
    return x, y, a, b


@pytest.mark.parametrize("n,m,d,eps,scale", [(5, 7, 2, 0.1, 1.0), (8, 3, 3, 0.05, 2.5), (1, 6, 1, 0.2, 1.0)])
def test_matches_bruteforce_scaling_iteration(rng, n, m, d, eps, scale):
    """Exp-domain Sinkhorn u = a/(K v), v = b/(K^T u), K = exp(-C/eps), is the
    same iteration in exact arithmetic: f = eps log(u/a), g = eps log(v/b)."""
    x, y, a, b = _clouds(rng, n, m, d)
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    C = scale * cdist(x.astype(np.float64), y.astype(np.float64), "sqeuclidean")
    K = np.exp(-C / eps)
    u, v = a64.copy(), b64.copy()  # f = g = 0
    f = np.zeros(n)
    g = np.zeros(m)
    for _ in range(25):
        u = a64 / (K @ v)
        v = b64 / (K.T @ u)
        f = oracle.halfstep_f(x, y, b, g, eps, scale)
        g = oracle.halfstep_g(x, y, a, f, eps, scale)
        np.testing.assert_allclose(f, eps * np.log(u / a64), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g, eps * np.log(v / b64), rtol=1e-11, atol=1e-12)
    # the plan built from scalings equals the oracle's plan
    P = u[:, None] * K * v[None, :]
    np.testing.assert_allclose(oracle.plan_rows(x, y, a, b, f, g, eps, scale), P, rtol=1e-10, atol=1e-15)


def test_single_point_is_the_single_mass():
    x = np.array([[0.3, -0.2]], np.float32)
    y = np.array([[1.1, 0.4]], np.float32)
    one = np.ones(1, np.float32)
    C = float(((x.astype(np.float64) - y.astype(np.float64)) ** 2).sum())
    for g0 in (0.0, 0.37, -5.0):
        f = oracle.halfstep_f(x, y, one, np.array([g0]), 0.05, 1.0)
        assert f[0] + g0 == pytest.approx(C, abs=1e-14)
        P = oracle.plan_rows(x, y, one, one, f, np.array([g0]), 0.05, 1.0)
        assert P[0, 0] == pytest.approx(1.0, abs=1e-12)


def test_halfstep_shift_and_plan_invariance(rng):
    x, y, a, b = _clouds(rng, 40, 30, 3)
    g = rng.normal(0, 0.05, size=30)
    f1 = oracle.halfstep_f(x, y, b, g, 0.02, 1.0)
    f2 = oracle.halfstep_f(x, y, b, g + 0.125, 0.02, 1.0)
    np.testing.assert_allclose(f2, f1 - 0.125, atol=1e-13)
    P1 = oracle.plan_rows(x, y, a, b, f1, g, 0.02, 1.0)
    P2 = oracle.plan_rows(x, y, a, b, f1 + 0.3, g - 0.3, 0.02, 1.0)
    np.testing.assert_allclose(P1, P2, rtol=1e-11)


def test_symmetric_problem_gives_equal_potentials_up_to_a_constant(rng):
    x = rng.uniform(0, 1, size=(30, 2)).astype(np.float32)
    a = np.full(30, 1 / 30, np.float32)
    res = oracle.solve(x, x, a, a, 1.0, Schedule(0.05, 0.05, tol=1e-12, max_iters=5000))
    assert res.converged
    diff = res.f - res.g
    assert np.ptp(diff) < 1e-9


def test_marginals_converge_and_primal_equals_dual(rng):
    x, y, a, b = _clouds(rng, 25, 35, 2)
    # float64 weights with equal sums: fp32 rounding of the two masses would
    # leave a residual floor of about 1e-8
    a = a.astype(np.float64) / a.astype(np.float64).sum()
    b = b.astype(np.float64) / b.astype(np.float64).sum()
    eps = 0.03
    res = oracle.solve(x, y, a, b, 1.0, Schedule(eps, eps, tol=1e-12, max_iters=20000))
    assert res.converged and max(res.R_row, res.R_col) <= 1e-12
    # independent check of the marginals from the scipy-built kernel
    C = cdist(x.astype(np.float64), y.astype(np.float64), "sqeuclidean")
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    P = a64[:, None] * b64[None, :] * np.exp((res.f[:, None] + res.g[None, :] - C) / eps)
    np.testing.assert_allclose(P.sum(1), a64, atol=1e-12)
    np.testing.assert_allclose(P.sum(0), b64, atol=1e-12)
    # primal <pi, C> + eps KL(pi | a x b) equals the dual <a, f> + <b, g>
    mu = a64[:, None] * b64[None, :]
    kl = float((P * np.log(P / mu) - P + mu).sum())
    primal = float((P * C).sum()) + eps * kl
    dual = float(a64 @ res.f + b64 @ res.g) - eps * float((P - mu).sum())
    assert primal == pytest.approx(dual, abs=1e-9)


def test_one_dimensional_entropic_cost_within_eps_log_n_of_sorted_w2(rng):
    """d = 1, uniform weights: W2^2 is the sorted matching, and
    W2^2 <= <pi_eps, C> <= W2^2 + eps log n (a permutation has KL = log n)."""
    n = 40
    x = rng.uniform(0, 1, size=(n, 1)).astype(np.float32)
    y = rng.normal(0.3, 0.3, size=(n, 1)).astype(np.float32)
    w = np.full(n, 1 / n, np.float32)
    eps = 0.01
    res = oracle.solve(x, y, w, w, 1.0, Schedule(1.0, eps, tol=1e-11, max_iters=50000))
    assert res.converged
    xs = np.sort(x[:, 0].astype(np.float64))
    ys = np.sort(y[:, 0].astype(np.float64))
    w2 = float(((xs - ys) ** 2).mean())
    P = oracle.plan_rows(x, y, w, w, res.f, res.g, eps, 1.0)
    C = (x.astype(np.float64) - y.astype(np.float64).T) ** 2
    cost = float((P * C).sum())
    assert w2 - 1e-9 <= cost <= w2 + eps * math.log(n) + 1e-9


def test_row_residual_identity_matches_explicit_plan(rng):
    x, y, a, b = _clouds(rng, 50, 45, 3)
    eps = 0.02
    f = rng.normal(0, 0.02, size=50)
    g = rng.normal(0, 0.02, size=45)
    f_next = oracle.halfstep_f(x, y, b, g, eps, 1.0)
    R_row, _ = oracle.marginal_residuals(x, y, a, b, f, g, eps, 1.0)
    assert oracle.row_residual_identity(a, f, f_next, eps) == pytest.approx(R_row, rel=1e-11)
    # right after a g half-step the columns are exact
    g_next = oracle.halfstep_g(x, y, a, f, eps, 1.0)
    _, R_col = oracle.marginal_residuals(x, y, a, b, f, g_next, eps, 1.0)
    assert R_col < 1e-14


def test_mean_cost_closed_form(rng):
    x, y, _, _ = _clouds(rng, 123, 77, 5)
    x64, y64 = x.astype(np.float64), y.astype(np.float64)
    closed = (x64 ** 2).sum(1).mean() + (y64 ** 2).sum(1).mean() - 2 * x64.mean(0) @ y64.mean(0)
    assert oracle.mean_sqeuclid(x, y) == pytest.approx(closed, rel=1e-12)


def test_all_minus_inf_lse_and_massless_targets():
    Z = np.array([[-np.inf, -np.inf], [0.0, -np.inf], [1.0, 1.0]])
    out = oracle.logsumexp_rows(Z)
    assert out[0] == -np.inf
    assert out[1] == 0.0
    assert out[2] == pytest.approx(1.0 + math.log(2.0))
    x = np.zeros((2, 1), np.float32)
    y = np.ones((3, 1), np.float32)
    f = oracle.halfstep_f(x, y, np.zeros(3, np.float32), np.zeros(3), 0.1, 1.0)
    assert np.all(f == np.inf)


def test_materialized_rows_sum_to_a_after_f_step_and_min_row_brute_force(rng):
    x, y, a, b = _clouds(rng, 30, 20, 2)
    a[3] = 0.0  # a massless row takes no part in min_row
    eps = 0.05
    g = rng.normal(0, 0.05, size=20)
    f = oracle.halfstep_f(x, y, b, g, eps, 1.0)
    rows = np.array([0, 3, 7, 29])
    T = oracle.materialize_rows(x, y, a, b, f, g, eps, 1.0, rows)
    np.testing.assert_allclose(T.sum(1), a[rows].astype(np.float64), rtol=1e-12, atol=1e-300)
    C = cdist(x.astype(np.float64), y.astype(np.float64), "sqeuclidean")
    u = a.astype(np.float64) * np.exp(f / eps)
    v = b.astype(np.float64) * np.exp(g / eps)
    P = u[:, None] * np.exp(-C / eps) * v[None, :]
    brute = min(P[i].max() for i in range(30) if a[i] > 0)
    assert oracle.min_row(x, y, a, b, f, g, eps, 1.0) == pytest.approx(brute, rel=1e-12)


def test_annealing_stage_counts():
    # eps 1 -> 1e-3 by halving: 1 ... 2^-9 (10 stages), then 1e-3
    assert len(oracle.annealing_stages(Schedule(1.0, 1e-3))) == 10
    # eps 1 -> 1e-4: 1 ... 2^-13 (14 stages), then 1e-4
    st = oracle.annealing_stages(Schedule(1.0, 1e-4))
    assert len(st) == 14 and st[-1] == 2.0 ** -13
    assert oracle.annealing_stages(Schedule(0.01, 0.01)) == []


def test_solve_fixed_iterations_counts(rng):
    x, y, a, b = _clouds(rng, 12, 9, 2)
    res = oracle.solve(x, y, a, b, 1.0, Schedule(0.01, 0.01, fixed_iters=7))
    assert res.iters == 7 and res.final_iters == 7
    res = oracle.solve(x, y, a, b, 1.0, Schedule(0.4, 0.1, iters_per_stage=3, fixed_iters=2))
    assert res.iters == 2 * 3 + 2


def test_sparsify_matches_a_scipy_csr_of_the_thresholded_plan(rng):
    """moscot #846: the kept entries are exactly the plan entries >= the
    threshold; scipy's CSR of the thresholded dense plan is the reference."""
    from scipy.sparse import csr_matrix

    x, y, a, b = _clouds(rng, 23, 31, 2)
    f = rng.normal(0, 0.01, 23)
    g = rng.normal(0, 0.01, 31)
    eps = 0.02
    P = oracle.plan_rows(x, y, a, b, f, g, eps, 1.0)
    thr = float(np.quantile(P, 0.8))
    ptr, col, val = oracle.sparsify(x, y, a, b, f, g, eps, 1.0, thr)
    ref = csr_matrix(np.where(P >= thr, P, 0.0))
    ref.sort_indices()
    np.testing.assert_array_equal(ptr, ref.indptr)
    np.testing.assert_array_equal(col, ref.indices)
    np.testing.assert_allclose(val, ref.data, rtol=0, atol=0)


def test_sparsify_at_min_row_keeps_every_row_with_mass(rng):
    x, y, a, b = _clouds(rng, 30, 26, 3)
    a = a.astype(np.float64)
    a[[3, 17]] = 0.0  # rows without mass: no entry, no part in the threshold
    f = rng.normal(0, 0.02, 30)
    g = rng.normal(0, 0.02, 26)
    eps = 0.01
    thr = oracle.min_row(x, y, a, b, f, g, eps, 1.0)
    ptr, col, val = oracle.sparsify(x, y, a, b, f, g, eps, 1.0, thr)
    per_row = np.diff(ptr)
    assert per_row[3] == 0 and per_row[17] == 0
    assert np.all(per_row[a > 0] >= 1)
    # the row that sets the threshold keeps exactly its largest entry
    P = oracle.plan_rows(x, y, a, b, f, g, eps, 1.0)
    i = int(np.argmin(np.where(a > 0, P.max(axis=1), np.inf)))
    assert per_row[i] >= 1 and val[ptr[i]:ptr[i + 1]].max() == P[i].max()
    # above the largest entry nothing survives
    ptr, col, val = oracle.sparsify(x, y, a, b, f, g, eps, 1.0, float(P.max()) * 1.5)
    assert ptr[-1] == 0 and len(col) == 0
