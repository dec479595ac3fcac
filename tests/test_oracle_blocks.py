"""Pins for the block screen and sparse half-steps: brute-force omitted-mass
bounds (FlashSinkhorn 2, §A.3), shift invariance, transposition, and the
reduction to the dense update when every tile is admitted."""
import math

import numpy as np
import pytest
from scipy.spatial.distance import cdist

import oracle
import synth


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


def _masked_plan_residual(P, Q, wp, wq, f, g, eps, M):
    """L1 residual of the rows of the plan restricted to the point mask M
    (scipy cdist for the cost, the plan written out entry by entry)."""
    C = cdist(P.astype(np.float64), Q.astype(np.float64), "sqeuclidean")
    pi = (wp.astype(np.float64)[:, None] * wq.astype(np.float64)[None, :]
          * np.exp((f.astype(np.float64)[:, None] + g.astype(np.float64)[None, :] - C) / eps))
    rows = np.where(M, pi, 0.0).sum(axis=1)
    return float(np.abs(rows - wp.astype(np.float64)).sum())


def test_sparse_residuals_equal_the_explicitly_masked_plan(problem):
    """FlashSinkhorn 2, §C.4: the certificate's residual is the one of the plan
    restricted to the admitted support. Built independently here: a block mask
    (with a row block and a column block that hold no tile, so both take the
    dense support), expanded to points with np.kron, and the plan from
    scipy's cdist."""
    x, y, a, b, f, g, eps = problem
    B = 32
    NB, MB = math.ceil(len(x) / B), math.ceil(len(y) / B)
    rng = np.random.default_rng(3)
    Mb = rng.random((NB, MB)) < 0.3
    Mb[2, :] = False  # row block 2: no admitted tile
    Mb[:, 5] = False  # column block 5: no admitted tile
    Mb[7, :] = True   # a full row block
    ptr = np.concatenate([[0], np.cumsum(Mb.sum(1))]).astype(np.int64)
    col = np.concatenate([np.nonzero(Mb[I])[0] for I in range(NB)]).astype(np.int32)
    ptrT = np.concatenate([[0], np.cumsum(Mb.sum(0))]).astype(np.int64)
    rowT = np.concatenate([np.nonzero(Mb[:, J])[0] for J in range(MB)]).astype(np.int32)
    Mp = np.kron(Mb, np.ones((B, B), bool))[:len(x), :len(y)]
    Mr = Mp.copy()
    Mr[~Mr.any(axis=1)] = True  # rows of a block without tiles: every column
    Mc = Mp.T.copy()
    Mc[~Mc.any(axis=1)] = True  # columns of a block without tiles: every row
    assert not Mr.all() and not Mc.all()
    want_row = _masked_plan_residual(x, y, a, b, f, g, eps, Mr)
    want_col = _masked_plan_residual(y, x, b, a, g, f, eps, Mc)
    Rr, Rc = oracle.sparse_residuals(x, y, a, b, f, g, eps, 1.0, ptr, col, ptrT, rowT, B)
    assert Rr == pytest.approx(want_row, rel=1e-12, abs=1e-15)
    assert Rc == pytest.approx(want_col, rel=1e-12, abs=1e-15)
    # the restriction matters here: the full-support residuals differ
    full_row = _masked_plan_residual(x, y, a, b, f, g, eps, np.ones_like(Mr))
    full_col = _masked_plan_residual(y, x, b, a, g, f, eps, np.ones_like(Mc))
    assert abs(full_row - want_row) > 1e-6 * want_row
    assert abs(full_col - want_col) > 1e-6 * want_col


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


# ---- tile verification (FlashSinkhorn 2, §3.2: exact B^2-pair mass of each candidate)

def _plan(x, y, a, b, f, g, eps):
    """The explicit plan pi from scipy's distance routine (not cost_rows)."""
    C = cdist(x.astype(np.float64), y.astype(np.float64), "sqeuclidean")
    return (a.astype(np.float64)[:, None] * b.astype(np.float64)[None, :]
            * np.exp((f.astype(np.float64)[:, None] + g.astype(np.float64)[None, :] - C) / eps))


def _verified(problem, B):
    x, y, a, b, f, g, eps = problem
    NB, MB = math.ceil(len(x) / B), math.ceil(len(y) / B)
    delta = 1e-3 / max(NB, MB)
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, delta)
    keep = oracle.verify_tiles(x, y, a, b, f, g, eps, 1.0, ptr, col, B, delta)
    return ptr, col, keep, delta, NB, MB


def test_tile_shares_match_the_explicit_plan(problem):
    x, y, a, b, f, g, eps = problem
    B = 32
    P = _plan(x, y, a, b, f, g, eps)
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    for I, J in [(0, 0), (3, 5), (19, 17), (7, 2)]:
        s, t = oracle.tile_shares(x, y, a, b, f, g, eps, 1.0, I, J, B)
        T = P[I * B:(I + 1) * B, J * B:(J + 1) * B]
        np.testing.assert_allclose(s, T.sum(axis=1) / a64[I * B:(I + 1) * B], rtol=1e-10, atol=1e-300)
        np.testing.assert_allclose(t, T.sum(axis=0) / b64[J * B:(J + 1) * B], rtol=1e-10, atol=1e-300)


def test_verification_keeps_exactly_the_tiles_with_a_large_share(problem):
    """Against brute force on the explicit plan: every candidate with some
    row share above delta a_i or column share above delta b_j is kept, every
    other candidate is dropped unless a fallback restores it."""
    x, y, a, b, f, g, eps = problem
    B = 32
    ptr, col, keep, delta, NB, MB = _verified(problem, B)
    P = _plan(x, y, a, b, f, g, eps)
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    big = np.zeros(len(col), bool)
    for I in range(NB):
        for e in range(ptr[I], ptr[I + 1]):
            J = int(col[e])
            T = P[I * B:(I + 1) * B, J * B:(J + 1) * B]
            big[e] = ((T.sum(axis=1) > delta * a64[I * B:(I + 1) * B]).any()
                      or (T.sum(axis=0) > delta * b64[J * B:(J + 1) * B]).any())
    assert (keep | ~big).all() and (keep >= big).all()
    restored = keep & ~big
    for e in np.nonzero(restored)[0]:
        I = int(np.searchsorted(ptr, e, side="right") - 1)
        J = int(col[e])
        row_none = not big[ptr[I]:ptr[I + 1]].any()
        col_none = not big[col == J].any()
        assert row_none or col_none, (I, J)
    assert 0 < keep.sum() < len(col)  # the workload drops some candidates and keeps some


def test_verification_keeps_the_omitted_mass_bound(problem):
    x, y, a, b, f, g, eps = problem
    B = 32
    ptr, col, keep, delta, NB, MB = _verified(problem, B)
    ptrV, colV, ptrT, rowsT = oracle.compact_tiles(ptr, col, keep, MB)
    M = _dense_mask(ptrV, colV, NB, MB)
    P = _plan(x, y, a, b, f, g, eps)
    mask = np.kron(M, np.ones((B, B), bool))[:len(x), :len(y)]
    omitted = np.where(mask, 0.0, P)
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    per_row_tiles = (~M).sum(axis=1)
    per_col_tiles = (~M).sum(axis=0)
    rows = np.repeat(np.arange(NB), B)[:len(x)]
    cols = np.repeat(np.arange(MB), B)[:len(y)]
    assert (omitted.sum(axis=1) <= delta * a64 * per_row_tiles[rows] * (1 + 1e-12)).all()
    assert (omitted.sum(axis=0) <= delta * b64 * per_col_tiles[cols] * (1 + 1e-12)).all()
    assert omitted.sum() <= max(NB, MB) * delta * (1 + 1e-12)


def test_single_point_blocks_verify_to_the_screen(rng):
    """With B = 1 the screen's bound is the plan entry itself, so the exact
    check agrees with it and drops no candidate (away from exact ties)."""
    x = rng.uniform(0, 1, (40, 2)).astype(np.float32)
    y = rng.uniform(0, 1, (35, 2)).astype(np.float32)
    a = np.full(40, 1 / 40, np.float32)
    b = np.full(35, 1 / 35, np.float32)
    eps = 0.01
    f, g = _potentials(x, y, a, b, eps, iters=20)
    delta = 1e-2 / 40
    sx = oracle.block_summaries(x, a, f, 1)
    sy = oracle.block_summaries(y, b, g, 1)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, delta)
    keep = oracle.verify_tiles(x, y, a, b, f, g, eps, 1.0, ptr, col, 1, delta)
    assert 0 < len(col) < 40 * 35 and keep.all()


def test_fallbacks_keep_blocks_that_would_lose_every_candidate(problem):
    x, y, a, b, f, g, eps = problem
    B = 32
    NB, MB = math.ceil(len(x) / B), math.ceil(len(y) / B)
    # every tile a candidate, threshold far above any share: all would go
    ptr = np.arange(NB + 1, dtype=np.int64) * MB
    col = np.tile(np.arange(MB, dtype=np.int32), NB)
    keep = oracle.verify_tiles(x, y, a, b, f, g, eps, 1.0, ptr, col, B, 10.0)
    assert keep.all()
    # row block 0 alone has candidates and all of them fail: kept by the
    # row fallback
    ptr1 = np.zeros(NB + 1, np.int64)
    ptr1[1:] = 3
    col1 = np.array([1, 4, MB - 1], np.int32)
    keep1 = oracle.verify_tiles(x, y, a, b, f, g, eps, 1.0, ptr1, col1, B, 10.0)
    assert keep1.all()
    # row block 0 has its heaviest tile J0 and a near-empty tile Jc; no other
    # row block has Jc. Verification drops (0, Jc), the row keeps J0, and the
    # column fallback restores (0, Jc) since column block Jc would lose all
    delta = 1e-3 / max(NB, MB)
    share = np.array([max(oracle.tile_shares(x, y, a, b, f, g, eps, 1.0, 0, J, B)[0].max(),
                          oracle.tile_shares(x, y, a, b, f, g, eps, 1.0, 0, J, B)[1].max())
                      for J in range(MB)])
    J0, Jc = int(np.argmax(share)), int(np.argmin(share))
    assert share[J0] > delta >= share[Jc]
    col2 = np.array(sorted([J0, Jc]), np.int32)
    ptr2 = np.zeros(NB + 1, np.int64)
    ptr2[1:] = 2
    keep2 = oracle.verify_tiles(x, y, a, b, f, g, eps, 1.0, ptr2, col2, B, delta)
    assert keep2.all()
    # with Jc also a (heavy) candidate of another row block, it is dropped
    # from row block 0
    Ih = int(np.argmax([oracle.tile_shares(x, y, a, b, f, g, eps, 1.0, I, Jc, B)[0].max()
                        for I in range(NB)]))
    assert Ih != 0
    assert oracle.tile_shares(x, y, a, b, f, g, eps, 1.0, Ih, Jc, B)[0].max() > delta
    ptr3 = np.zeros(NB + 1, np.int64)
    ptr3[1:Ih + 1] = 2
    ptr3[Ih + 1:] = 3
    col3 = np.concatenate([col2, np.array([Jc], np.int32)])
    keep3 = oracle.verify_tiles(x, y, a, b, f, g, eps, 1.0, ptr3, col3, B, delta)
    assert list(keep3) == [J0 < Jc, J0 > Jc, True]


def test_compacted_lists_are_transposes(problem):
    B = 32
    ptr, col, keep, delta, NB, MB = _verified(problem, B)
    ptrV, colV, ptrT, rowsT = oracle.compact_tiles(ptr, col, keep, MB)
    M = _dense_mask(ptrV, colV, NB, MB)
    MT = _dense_mask(ptrT, rowsT, MB, NB)
    assert (M == MT.T).all()
    assert ptrV[-1] == keep.sum() == ptrT[-1]
    for J in range(MB):
        r = rowsT[ptrT[J]:ptrT[J + 1]]
        assert (np.diff(r) > 0).all()


def test_process_pool_screen_digests_equal_the_single_process_screen():
    """The full-size GPU checks compare tile lists against the oracle's screen
    run over worker processes by row-block ranges: those digests must be the
    single-process screen's, range by range."""
    import oracle_pool

    n, B, eps = 16384, 128, 1e-3
    c = synth.make(5, n=n, m=n)
    _, px, _, py = oracle.morton_order(c.x, c.y)
    x, y, a, b = c.x[px], c.y[py], c.a[px], c.b[py]
    rng = np.random.default_rng(4)
    base = eps * math.log(n) / 2
    f = (base + rng.normal(0, 0.3 * eps, n)).astype(np.float32)
    g = (base + rng.normal(0, 0.3 * eps, n)).astype(np.float32)
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    delta = 1e-3 / (n // B)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, delta)
    assert 0 < len(col) < (n // B) ** 2
    got = oracle_pool.screen_digests(sx, sy, eps, 1.0, delta, width=24, procs=2)
    assert [(lo, hi) for lo, hi, _, _ in got] == oracle_pool.spans(n // B, 24)
    for lo, hi, counts, h in got:
        want_counts, want_h = oracle_pool.digest(ptr, col, lo, hi)
        assert np.array_equal(counts, want_counts) and h == want_h
    # a single changed tile index changes its range's digest
    col2 = col.copy()
    col2[len(col2) // 2] ^= 1
    assert any(oracle_pool.digest(ptr, col2, lo, hi)[1] != h for lo, hi, _, h in got)
