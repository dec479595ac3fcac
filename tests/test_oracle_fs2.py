"""Pins for cells, the lift and the multiscale pipeline.

The lift is pinned by the worked example of FlashSinkhorn 2, §A.1 (proof of
Proposition 1): two-point clouds at -h and +h collapsed into one cell have zero
coarse potentials, and the lifted potentials give L1 residual cosh(2h^2/eps) - 1.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.fs2 import FS2Params

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lift_cosh.json")


def test_cosh_worked_example():
    with open(GOLDEN) as fh:
        cases = json.load(fh)["cases"]
    for case in cases:
        h, eps = case["h"], case["eps"]
        pts = np.array([[-h], [h]], np.float32)
        w = np.array([0.5, 0.5], np.float32)
        codes, perm, _, _ = oracle.morton_order(pts, pts)
        off, cent, mass = oracle.cells(codes, pts[perm], w[perm], 0)  # one cell per side
        assert len(mass) == 1 and mass[0] == 1.0 and cent[0, 0] == 0.0
        # the coarse problem is one point against one point: F = G = 0
        F = oracle.halfstep_f(cent, cent, mass, np.zeros(1), eps, 1.0)
        assert F[0] == 0.0
        f = oracle.lift(pts, cent, mass, np.zeros(1), eps, 1.0)
        g = oracle.lift(pts, cent, mass, np.zeros(1), eps, 1.0)
        h2 = float(np.float32(h)) ** 2
        np.testing.assert_allclose(f, [h2, h2], rtol=1e-14)
        R_row, R_col = oracle.marginal_residuals(pts, pts, w, w, f, g, eps, 1.0)
        expected = math.cosh(2 * h2 / eps) - 1.0
        assert R_row == pytest.approx(expected, rel=1e-12)
        assert R_col == pytest.approx(expected, rel=1e-12)
        assert case["cosh_arg"] == pytest.approx(2 * h * h / eps, rel=1e-6)


def test_singleton_cells_make_the_lift_an_ordinary_halfstep(rng):
    x = rng.uniform(0, 1, size=(64, 3)).astype(np.float32)
    y = rng.uniform(0, 1, size=(50, 3)).astype(np.float32)
    b = np.full(50, 1 / 50, np.float32)
    cx, px, cy, py = oracle.morton_order(x, y)
    off, cent, mass = oracle.cells(cy, y[py], b[py], 63)
    assert len(mass) == 50
    G = rng.normal(0, 0.01, size=50)
    f = oracle.lift(x, cent, mass, G, 0.01, 1.0)
    np.testing.assert_allclose(f, oracle.halfstep_f(x, y[py], b[py], G, 0.01, 1.0), rtol=1e-12)


def test_cells_partition_and_centroids(rng):
    x = rng.uniform(0, 1, size=(500, 3)).astype(np.float32)
    w = rng.uniform(0, 1, size=500).astype(np.float32)
    cx, px, _, _ = oracle.morton_order(x, x)
    off, cent, mass = oracle.cells(cx, x[px], w[px], 6)
    assert off[0] == 0 and off[-1] == 500 and np.all(np.diff(off) > 0)
    assert len(mass) <= 64
    assert mass.sum() == pytest.approx(w.astype(np.float64).sum(), rel=1e-12)
    xs, ws = x[px].astype(np.float64), w[px].astype(np.float64)
    for c in range(len(mass)):
        s, e = off[c], off[c + 1]
        # every point of a cell shares the top 6 code bits, i.e. a 4x4x4 octree box
        assert len(set((cx[s:e] >> np.uint64(57)).tolist())) == 1
        np.testing.assert_allclose(cent[c], (ws[s:e, None] * xs[s:e]).sum(0) / ws[s:e].sum(), rtol=1e-12)


@pytest.mark.parametrize("verify", [False, True], ids=["screened", "verified"])
def test_pipeline_is_certified_and_the_certificate_holds(rng, verify):
    cx = rng.uniform(0.2, 0.8, size=(4, 3))
    n = 2048
    lab = rng.integers(0, 4, n)
    x = (cx[lab] + rng.normal(0, 0.03, size=(n, 3))).astype(np.float32)
    y = (cx[lab] + rng.normal(0, 0.03, size=(n, 3)) + 0.01).astype(np.float32)
    w = np.full(n, 1 / n, np.float32)
    prm = FS2Params(B=64, eps=2e-3, tol=2e-2, max_fine=60, verify=verify)
    res = oracle.fs2_solve(x, y, w, w, prm)
    assert res.certified
    if verify:  # verification drops some screened tiles
        assert res.tiles_history[-1] < res.candidates_history[-1]
    Fr, Fc = oracle.marginal_residuals(x, y, w, w, res.f, res.g, prm.eps, 1.0)
    assert max(Fr, Fc) <= prm.tol
    assert max(Fr, Fc) <= max(res.R_A_row, res.R_A_col) + res.omega + 1e-12


# ---- sampled lift checks and the adaptive coarse-to-fine switch (FlashSinkhorn 2, §3.1, §B.2)

from oracle.fs2 import lift_accepted, sample_indices, sampled_residual  # noqa: E402


def test_sample_indices_range_reuse_and_uniformity():
    a = sample_indices(1000, 8192, 7, 0)
    assert a.dtype == np.int64 and a.min() >= 0 and a.max() < 1000
    assert np.array_equal(sample_indices(1000, 1024, 7, 0), a[:1024])  # the first draws are reused
    assert not np.array_equal(sample_indices(1000, 1024, 7, 1), a[:1024])  # other side, other stream
    counts = np.bincount(sample_indices(10, 200000, 3, 0), minlength=10)
    chi2 = float(((counts - 20000.0) ** 2 / 20000.0).sum())
    assert chi2 < 40.0  # 9 degrees of freedom: p ~ 1e-5


def _small_problem(rng, n=600, eps=0.02, iters=5):
    x = rng.uniform(0, 1, (n, 2)).astype(np.float32)
    y = rng.uniform(0, 1, (n, 2)).astype(np.float32)
    a = rng.uniform(0.5, 1.5, n)
    a = (a / a.sum()).astype(np.float32)
    b = np.full(n, 1.0 / n, np.float32)
    res = oracle.solve(x, y, a, b, 1.0, oracle.Schedule(eps, eps, fixed_iters=iters))
    return x, y, a, b, res.f, res.g, eps


def test_sampled_residual_with_every_row_once_is_the_residual(rng):
    x, y, a, b, f, g, eps = _small_problem(rng)
    R_row, R_col = oracle.marginal_residuals(x, y, a, b, f, g, eps, 1.0)
    est, se = sampled_residual(x, y, a, b, f, g, eps, 1.0, np.arange(len(x)))
    assert est == pytest.approx(R_row, rel=1e-12)
    est_c, _ = sampled_residual(y, x, b, a, g, f, eps, 1.0, np.arange(len(y)))
    assert est_c == pytest.approx(R_col, rel=1e-12, abs=1e-15)


def test_sampled_residual_is_unbiased_and_its_error_is_the_sample_spread(rng):
    x, y, a, b, f, g, eps = _small_problem(rng)
    R_row, _ = oracle.marginal_residuals(x, y, a, b, f, g, eps, 1.0)
    ests, ses = [], []
    for seed in range(40):
        e, s = sampled_residual(x, y, a, b, f, g, eps, 1.0, sample_indices(len(x), 64, seed, 0))
        ests.append(e)
        ses.append(s)
    # the mean of 40 independent estimates sits within 4 of its standard errors
    assert abs(np.mean(ests) - R_row) < 4.0 * np.mean(ses) / math.sqrt(40)
    # and the reported standard error matches the spread of the estimates
    assert 0.5 < np.std(ests, ddof=1) / np.mean(ses) < 1.6
    # a residual that is the same on every row has no spread
    f0 = f.copy()
    est, se = sampled_residual(x, y, a, b, f0, g, eps, 1.0, np.zeros(16, np.int64))
    assert se == 0.0


def test_adaptive_switch_accepts_an_exact_lift(rng):
    """Singleton cells make the lift an ordinary half-step, so after enough
    centroid updates the lifted potentials pass the sampled check and are
    returned without fine updates; their exact residual is under tol."""
    n = 512
    x = rng.uniform(0, 1, (n, 2)).astype(np.float32)
    y = rng.uniform(0, 1, (n, 2)).astype(np.float32)
    w = np.full(n, 1.0 / n, np.float32)
    prm = FS2Params(B=16, eps=0.005, tol=1e-2, p_bits=42, coarse_tol=0.0, stall_window=1 << 30,
                    coarse_iters_per_stage=2, adaptive=True, check_every=3, check_samples=128,
                    check_samples_max=512)
    res = oracle.fs2_solve(x, y, w, w, prm)
    assert res.accepted_by_sample and res.fine_updates == 0 and not res.certified
    assert res.ncells_x == n and res.ncells_y == n
    R = max(oracle.marginal_residuals(x, y, w, w, res.f, res.g, prm.eps, 1.0))
    assert R < prm.tol
    er, sr, ec, sc, k = res.check_history[-1]
    assert max(er + 3 * sr, ec + 3 * sc) < prm.tol
    assert res.checks > 1  # earlier lifts failed the check
    er, sr, ec, sc, k = res.check_history[-2]
    assert max(er + 3 * sr, ec + 3 * sc) >= prm.tol
    # a check whose interval straddled tol was repeated with the larger sample
    assert any(h[4] == prm.check_samples_max for h in res.check_history)


def test_adaptive_switch_falls_back_to_certified_fine_updates(rng):
    cx = rng.uniform(0.2, 0.8, size=(4, 3))
    n = 2048
    lab = rng.integers(0, 4, n)
    x = (cx[lab] + rng.normal(0, 0.03, size=(n, 3))).astype(np.float32)
    y = (cx[lab] + rng.normal(0, 0.03, size=(n, 3)) + 0.01).astype(np.float32)
    w = np.full(n, 1 / n, np.float32)
    prm = FS2Params(B=64, eps=2e-3, tol=2e-2, max_fine=60, adaptive=True, check_every=32)
    res = oracle.fs2_solve(x, y, w, w, prm)
    assert not res.accepted_by_sample and res.checks >= 1 and res.certified and res.fine_updates > 0
    Fr, Fc = oracle.marginal_residuals(x, y, w, w, res.f, res.g, prm.eps, 1.0)
    assert max(Fr, Fc) <= max(res.R_A_row, res.R_A_col) + res.omega + 1e-12


# ---- the coarse stop rule and the cell prefix (FlashSinkhorn 2, §3, §3.1, §B.1, §B.2)

from oracle.fs2 import coarse_done, coarse_solve, prefix_bits  # noqa: E402


def _stop_after(history, prm):
    """Number of centroid updates run when the residuals come out as `history`."""
    for k in range(1, len(history) + 1):
        if coarse_done(history[:k], prm):
            return k
    return None


def test_coarse_stop_rule_on_hand_made_histories():
    prm = FS2Params(coarse_tol=1e-3, stall_window=10, stall_rel=0.01)
    # tolerance: stops at the first residual <= coarse_tol (equality included)
    assert _stop_after([0.5, 0.01, 0.0009, 0.0001], prm) == 3
    assert _stop_after([0.5, 1e-3], prm) == 2
    # a plateau at 0.2 after 1, 0.5, 0.25: the window of ten updates first
    # compares 0.2 with 1.0 (update 11), 0.5 (12), 0.25 (13: 0.2 <= 0.2475),
    # then with 0.2 itself at update 14 (0.2 > 0.198): stall
    assert _stop_after([1.0, 0.5, 0.25] + [0.2] * 30, prm) == 14
    # 0.05% less per update: 0.5% over ten updates, stalls as soon as the
    # window is full (update 11: 0.9945 > 0.99 * 0.9995)
    assert _stop_after([1.0 - 0.0005 * k for k in range(1, 40)], prm) == 11
    # exactly 1% less over the window is progress (stall needs more than 1 - stall_rel)
    assert _stop_after([1.0] + [0.995] * 9 + [0.99, 0.99], prm) == 12
    # 20% less per update never stalls and reaches the tolerance at 0.8^31 < 1e-3 (update 32)
    hist = [0.8 ** k for k in range(1, 60)]
    assert _stop_after(hist, prm) == 31
    assert 0.8 ** 30 > 1e-3 >= 0.8 ** 31


def test_coarse_stage_runs_the_annealing_then_at_most_coarse_max_updates(rng):
    x = rng.uniform(0, 1, size=(12, 2))
    y = rng.uniform(0, 1, size=(9, 2))
    mx = np.full(12, 1 / 12)
    my = np.full(9, 1 / 9)
    # stages 1, 0.5, 0.25, 0.125 above eps = 0.1, two updates each, then the cap of 3
    prm = FS2Params(eps=0.1, coarse_eps_start=1.0, coarse_factor=0.5, coarse_iters_per_stage=2,
                    coarse_tol=0.0, coarse_max=3, stall_window=1 << 30)
    _, _, iters = coarse_solve(x, y, mx, my, prm)
    assert iters == 4 * 2 + 3


def test_prefix_bits_give_at_most_twice_as_many_cells_as_blocks(rng):
    assert prefix_bits(131072, 131072, 3) == 18  # 2^24 points in blocks of 128
    assert prefix_bits(1, 1, 3) == 1
    assert prefix_bits(3, 2, 3) == 2  # 2^2 <= 6 < 2^3
    assert prefix_bits(4, 1, 3) == 3
    assert prefix_bits(1 << 40, 1, 1) == 21  # at most the code length
    for n in (300, 1000, 5000):
        x = rng.uniform(0, 1, size=(n, 3)).astype(np.float32)
        codes, perm, _, _ = oracle.morton_order(x, x)
        NB = (n + 127) // 128
        p = prefix_bits(NB, NB, 3)
        off, _, _ = oracle.cells(codes, x[perm], np.full(n, 1 / n, np.float32), p)
        assert len(off) - 1 <= 2 * NB
        assert 2 ** p <= 2 * NB < 2 ** (p + 1)
