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
