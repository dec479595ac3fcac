"""GPU parity of the block-sparse path against the fp64 oracle: Morton codes
and order and the block-pair tile lists bit-exact on identical inputs; sparse
half-steps within 1e-5 max(eps, |f|); the multiscale solve certified."""
import math
import os
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def sk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import log_domain_sinkhorn_amd as sk

    return sk


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _gpu_morton(sk, x, y):
    cx, px, cy, py = sk.morton_order(_t(x), _t(y))
    u = lambda c: c.cpu().numpy().view(np.uint64)
    return u(cx), px.cpu().numpy(), u(cy), py.cpu().numpy()


@pytest.mark.parametrize("w,n,m", [(5, None, None), (5, 5000, 3001), (4, 1000, 1000), (1, 999, 1001)])
def test_morton_codes_and_order_bit_exact(sk, w, n, m):
    c = synth.make(w, n=n, m=m)
    x, y = c.x, c.y
    if n == 5000:  # duplicates must keep their input order
        x = x.copy()
        x[100:200] = x[7]
    _log(f"morton w={w} n={len(x)}")
    got = _gpu_morton(sk, x, y)
    ref = oracle.morton_order(x, y)
    for g_, r_, what in zip(got, ref, ("codes_x", "perm_x", "codes_y", "perm_y")):
        assert np.array_equal(g_, r_), what


@pytest.mark.parametrize("w,n,m", [(5, 5000, 4321), (2, 1, 7), (1, 3001, 517)])
def test_handle_morton_sort_equals_the_standalone_order(sk, w, n, m):
    """The handle form (one side of a handle's clouds) gives the oracle's codes
    and order bit for bit, like the standalone call over both clouds."""
    c = synth.make(w, n=n, m=m)
    ref = oracle.morton_order(c.x, c.y)
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        cx, px = P.morton_sort(0)
        cy, py = P.morton_sort(1)
    got = (cx.cpu().numpy().view(np.uint64), px.cpu().numpy(), cy.cpu().numpy().view(np.uint64),
           py.cpu().numpy())
    for g_, r_, what in zip(got, ref, ("codes_x", "perm_x", "codes_y", "perm_y")):
        assert np.array_equal(g_.astype(np.int64) if what.startswith("perm") else g_,
                              r_.astype(np.int64) if what.startswith("perm") else r_), what


def _sorted_problem(w, n, seed_shift=0.0):
    c = synth.make(w, n=n, m=n)
    _, px, _, py = oracle.morton_order(c.x, c.y)
    return c.x[px], c.y[py], c.a[px], c.b[py]


def _near_plan_potentials(n, eps, rng):
    """f = g ~ eps log(n)/2 (+ noise): near pairs carry mass ~ 1/n, so the mask
    is neither empty nor full."""
    base = eps * math.log(n) / 2
    f = (base + rng.normal(0, 0.3 * eps, n)).astype(np.float32)
    g = (base + rng.normal(0, 0.3 * eps, n)).astype(np.float32)
    return f, g


@pytest.mark.parametrize("n,B,eps", [(65536, 128, 1e-4), (16384, 256, 1e-3), (5000, 128, 1e-3)])
def test_block_screen_bit_exact(sk, n, B, eps):
    x, y, a, b = _sorted_problem(5, n)
    rng = np.random.default_rng(1)
    f, g = _near_plan_potentials(n, eps, rng)
    NB = (n + B - 1) // B
    delta = 1e-3 / NB
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    ptr_r, col_r = oracle.screen(sx, sy, eps, 1.0, delta)
    ptrT_r, rowT_r = oracle.screen_transpose(sx, sy, eps, 1.0, delta)
    assert 0 < len(col_r) < NB * NB
    with sk.Problem(_t(x), _t(y), _t(a), _t(b), 1.0) as P:
        ptr, idx = P.block_screen(eps, _t(f), _t(g), B, delta)
        ptrT, idxT = P.block_screen(eps, _t(f), _t(g), B, delta, transpose=True)
    assert np.array_equal(ptr.cpu().numpy(), ptr_r) and np.array_equal(idx.cpu().numpy(), col_r)
    assert np.array_equal(ptrT.cpu().numpy(), ptrT_r) and np.array_equal(idxT.cpu().numpy(), rowT_r)


def test_block_screen_full_size_sampled_row_blocks(sk):
    """2^24 points, B = 128: every row block screened on the GPU against all
    131072 column blocks; 24 sampled row blocks recomputed by the oracle."""
    c = synth.make(5)
    cx, px, cy, py = _gpu_morton(sk, c.x, c.y)
    x, y, a, b = c.x[px], c.y[py], c.a[px], c.b[py]
    eps = 1e-4
    rng = np.random.default_rng(2)
    f, g = _near_plan_potentials(c.n, eps, rng)
    B = 128
    NB = c.n // B
    delta = 1e-3 / NB
    _log("screen full size")
    with sk.Problem(_t(x), _t(y), None, None, 1.0) as P:
        ptr, idx = P.block_screen(eps, _t(f), _t(g), B, delta)
    ptr = ptr.cpu().numpy()
    idx = idx.cpu().numpy()
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    rows = np.sort(rng.choice(NB, 24, replace=False))
    ptr_r, col_r = oracle.screen(sx, sy, eps, 1.0, delta, row_blocks=rows)
    for k, I in enumerate(rows):
        assert np.array_equal(idx[ptr[I]:ptr[I + 1]], col_r[ptr_r[k]:ptr_r[k + 1]]), I


def test_block_screen_capacity_overflow_reports_the_needed_count(sk):
    """A tile-list capacity one short of the need: SINKHORN_ERR_CAPACITY,
    the needed count in nnz_out, the index array left unwritten."""
    import ctypes

    n, B, eps = 5000, 128, 1e-3
    x, y, a, b = _sorted_problem(5, n)
    f, g = _near_plan_potentials(n, eps, np.random.default_rng(5))
    delta = 1e-3 / ((n + B - 1) // B)
    with sk.Problem(_t(x), _t(y), _t(a), _t(b), 1.0) as P:
        fd, gd = _t(f), _t(g)
        _, idx = P.block_screen(eps, fd, gd, B, delta)
        need = int(idx.shape[0])
        assert need > 1
        ptr = torch.empty((n + B - 1) // B + 1, dtype=torch.int64, device=DEV)
        small = torch.full((need - 1,), -7, dtype=torch.int32, device=DEV)
        nnz = ctypes.c_int64(-1)
        code = sk.lib().sinkhorn_block_screen(P._h, eps, sk._ptr(fd), sk._ptr(gd), B, delta, 0,
                                              sk._ptr(ptr), sk._ptr(small), need - 1, ctypes.byref(nnz))
        assert code == sk.ERR_CAPACITY and nnz.value == need
        assert bool((small == -7).all())
        assert b"capacity" in sk.lib().sinkhorn_strerror(code)


def test_sparse_halfstep_with_weights_beyond_fp32_range(sk):
    """Column weights 2^-130 below the rest (subnormal in fp32): a block whose
    tile-local weights would leave the normal fp32 range takes the difference
    form, and the shifted sparse f-step still matches the oracle."""
    n, B, eps = 16384, 128, 1e-3
    x, y, a, b = _sorted_problem(5, n)
    b = b.astype(np.float64)
    b[5::97] *= 2.0 ** -130
    b = (b * (a.astype(np.float64).sum() / b.sum())).astype(np.float32)  # balanced masses
    assert (b > 0).all() and (b[5::97] < np.finfo(np.float32).tiny).all()
    rng = np.random.default_rng(4)
    f, g = _near_plan_potentials(n, eps, rng)
    NB = (n + B - 1) // B
    delta = 1e-3 / NB
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, delta)
    with sk.Problem(_t(x), _t(y), _t(a), _t(b), 1.0) as P:
        fo, _ = P.sparse_halfstep_f(eps, _t(g), B, _t(ptr), _t(col.astype(np.int32)), f_prev=_t(f))
    ref = oracle.sparse_halfstep_f(x, y, b, g, eps, 1.0, ptr, col, B)
    err = np.abs(fo.cpu().numpy().astype(np.float64) - ref) / np.maximum(eps, np.abs(ref))
    assert err.max() <= 1e-5, err.max()


@pytest.mark.parametrize("prev", [True, False], ids=["shifted", "exact"])
@pytest.mark.parametrize("n,B,eps", [(16384, 128, 1e-4), (16384, 256, 1e-3), (5000, 128, 1e-3)])
def test_sparse_halfsteps_match_oracle(sk, n, B, eps, prev):
    """With the previous potentials the kernel runs the shifted loop (and
    reports the residual); without, the exact loop."""
    x, y, a, b = _sorted_problem(5, n)
    rng = np.random.default_rng(3)
    f, g = _near_plan_potentials(n, eps, rng)
    NB = (n + B - 1) // B
    delta = 1e-3 / NB
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, delta)
    ptrT, rowT = oracle.screen_transpose(sx, sy, eps, 1.0, delta)
    # force one empty row block so the dense fallback is exercised
    ptr = ptr.copy()
    col = np.delete(col, np.s_[ptr[1]:ptr[2]])
    ptr[2:] -= ptr[2] - ptr[1]
    with sk.Problem(_t(x), _t(y), _t(a), _t(b), 1.0) as P:
        fo, r = P.sparse_halfstep_f(eps, _t(g), B, _t(ptr), _t(col.astype(np.int32)),
                                    f_prev=_t(f) if prev else None)
        go, rc = P.sparse_halfstep_g(eps, _t(f), B, _t(ptrT), _t(rowT.astype(np.int32)),
                                     g_prev=_t(g) if prev else None)
    f_ref = oracle.sparse_halfstep_f(x, y, b, g, eps, 1.0, ptr, col, B)
    g_ref = oracle.sparse_halfstep_g(x, y, a, f, eps, 1.0, ptrT, rowT, B)
    for got, ref, what in ((fo, f_ref, "f"), (go, g_ref, "g")):
        got = got.cpu().numpy().astype(np.float64)
        err = np.abs(got - ref) / np.maximum(eps, np.abs(ref))
        assert err.max() <= 1e-5, (what, err.max())
    if prev:
        Rr, Rc = oracle.sparse_residuals(x, y, a, b, f, g, eps, 1.0, ptr, col, ptrT, rowT, B)
        assert r == pytest.approx(Rr, rel=1e-3) and rc == pytest.approx(Rc, rel=1e-3)
    else:
        assert r is None and rc is None


@pytest.mark.parametrize("offset", [0.0, 300.0, -300.0, "mixed"])
@pytest.mark.parametrize("eps", [1e-2, 1e-3])
def test_sparse_shifted_loop_matches_oracle_for_any_shift_estimate(sk, eps, offset):
    """The shifted sparse loop takes most tiles in the tile-local expanded
    form at these eps (the rest in the difference form). Its per-row shift
    comes from the previous potential: a good estimate, one far too low (tile
    sums pass 2^64: the shift moves up), one far too high (row sums underflow:
    exact recompute of the tile) and a mixture must all give the oracle's
    potentials within 1e-5 max(eps, |f|)."""
    n, B = 16384, 128
    x, y, a, b = _sorted_problem(5, n)
    rng = np.random.default_rng(17)
    f, g = _near_plan_potentials(n, eps, rng)
    NB = n // B
    delta = 1e-3 / NB
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, delta)
    f_ref = oracle.sparse_halfstep_f(x, y, b, g, eps, 1.0, ptr, col, B)
    if offset == "mixed":
        prev = f_ref + rng.choice([-300.0, 0.0, 300.0], n) * eps
    else:
        prev = f_ref + offset * eps
    with sk.Problem(_t(x), _t(y), _t(a), _t(b), 1.0) as P:
        fo, _ = P.sparse_halfstep_f(eps, _t(g), B, _t(ptr), _t(col.astype(np.int32)),
                                    f_prev=_t(prev.astype(np.float32)))
    got = fo.cpu().numpy().astype(np.float64)
    err = np.abs(got - f_ref) / np.maximum(eps, np.abs(f_ref))
    assert err.max() <= 1e-5, err.max()


def _gauge_close(f, g, fr, gr, tol):
    """Potentials equal up to the common shift (f + c, g - c), which leaves the
    plan unchanged (FlashSinkhorn 2, §A.3) and which fp32 rounding walks."""
    f = f.cpu().numpy().astype(np.float64)
    g = g.cpu().numpy().astype(np.float64)
    c = float(np.mean(f - fr))
    df = np.abs(f - c - fr).max()
    dg = np.abs(g + c - gr).max()
    assert df <= tol and dg <= tol, (df, dg, c, tol)


def test_multiscale_fixed_budget_matches_the_oracle(sk):
    """Cells, an all-iterations coarse stage, the lift and exactly four fine
    updates: same cell counts, iteration counts and (gauge-fixed) potentials
    within 1e-3 eps; the admitted residual of the returned state agrees."""
    path = os.path.join(GOLDEN, "fs2_w5_n16384_fixed.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing {path}: run tests/golden/make_solve_refs.py w5_n16384_fixed")
    ref = dict(np.load(path))
    n = int(ref["n"])
    c = synth.make(5, n=n, m=n)
    eps = float(ref["eps"])
    prm = sk.MultiscaleParams(B=int(ref["B"]), eps=eps, tol=float(ref["tol"]), coarse_tol=float(ref["coarse_tol"]),
                              coarse_max=int(ref["coarse_max"]), stall_window=int(ref["stall_window"]),
                              max_fine=int(ref["max_fine"]))
    _log(f"multiscale fixed budget n={n}")
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        f, g, rep = P.solve_multiscale(prm)
    assert rep["status"] == sk.NOT_CONVERGED and rep["certified"] == 0
    assert rep["ncells_x"] == int(ref["ncells_x"]) and rep["ncells_y"] == int(ref["ncells_y"])
    assert rep["coarse_iters"] == int(ref["coarse_iters"])
    assert rep["fine_updates"] == int(ref["fine_updates"]) == prm.max_fine
    # the mask is rebuilt from fp32 block maxima on both sides: a tile whose
    # mass bound sits at the threshold may flip, nothing more
    tiles = int(ref["tiles"][-1])
    assert abs(rep["last_tiles"] - tiles) <= max(2, tiles // 1000), (rep["last_tiles"], tiles)
    _gauge_close(f, g, ref["f"], ref["g"], 1e-3 * eps)
    assert rep["R_A_row"] == pytest.approx(float(ref["R_A_row"]), rel=1e-2)


def test_multiscale_warm_start_continues_the_fine_loop_bit_for_bit(sk):
    """A warm-started solve (no cells, coarse stage or lift) from the state an
    earlier solve returned continues its fine loop exactly: 2 updates, then 3
    more from the returned potentials, equal 5 updates in one call bit for
    bit; with no update allowed the potentials come back unchanged and the
    admitted residual is the one the first call reported."""
    n = 16384
    c = synth.make(5, n=n, m=n)
    base = dict(B=128, eps=1e-3, tol=1e-30, coarse_tol=0.0, coarse_max=40, stall_window=1 << 30)
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        f5, g5, r5 = P.solve_multiscale(sk.MultiscaleParams(**base, max_fine=5))
        f2, g2, r2 = P.solve_multiscale(sk.MultiscaleParams(**base, max_fine=2))
        f0, g0, r0 = P.solve_multiscale(sk.MultiscaleParams(**base, max_fine=0, warm_start=True),
                                        f2.clone(), g2.clone())
        assert torch.equal(f0, f2) and torch.equal(g0, g2)
        assert r0["R_A_row"] == r2["R_A_row"] and r0["ncells_x"] == 0 and r0["coarse_iters"] == 0
        fw, gw, rw = P.solve_multiscale(sk.MultiscaleParams(**base, max_fine=3, warm_start=True),
                                        f2.clone(), g2.clone())
    assert rw["status"] == sk.NOT_CONVERGED and rw["fine_updates"] == 3
    assert torch.equal(fw, f5) and torch.equal(gw, g5)
    assert rw["R_A_row"] == r5["R_A_row"] and rw["last_tiles"] == r5["last_tiles"]


@pytest.mark.parametrize("verify", [False, True], ids=["screened", "verified"])
def test_multiscale_solve_certificate_holds(sk, verify):
    """Run to the stop rule; the oracle's exact dense residuals of the returned
    potentials must sit under the certificate R_A + Omega <= tol."""
    n, eps = 16384, 1e-3
    c = synth.make(5, n=n, m=n)
    prm = sk.MultiscaleParams(B=128, eps=eps, tol=1e-2, verify=verify)
    _log(f"multiscale certified n={n} verify={verify}")
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        f, g, rep = P.solve_multiscale(prm)
    _log(f"  coarse {rep['coarse_iters']} fine {rep['fine_updates']} R_A {rep['R_A_row']:.3e}/{rep['R_A_col']:.3e}")
    assert rep["status"] == sk.OK and rep["certified"] == 1
    assert max(rep["R_A_row"], rep["R_A_col"]) + rep["omega"] <= prm.tol
    Fr, Fc = oracle.marginal_residuals(c.x, c.y, c.a, c.b, f.cpu().numpy(), g.cpu().numpy(), eps, 1.0)
    # fp32 potentials carry 1e-5 max(eps, |f|) / eps relative error into each row's mass
    fl = 1e-5 * max(1.0, float(np.abs(f.cpu().numpy()).max()) / eps)
    assert max(Fr, Fc) <= max(rep["R_A_row"], rep["R_A_col"]) + rep["omega"] + fl, (Fr, Fc, rep)


def _dense_check(sk, P, rep, eps, f, g, tol):
    """The certificate against the exact dense residuals of the returned
    potentials (every pair, fp64 sums on the GPU; parity-tested against the
    oracle in test_gpu_dense)."""
    assert rep["status"] == sk.OK and rep["certified"] == 1
    R_A = max(rep["R_A_row"], rep["R_A_col"])
    assert R_A + rep["omega"] <= tol
    Rr, Rc = P.marginal_residual(eps, f, g)
    _log(f"  certificate {R_A:.6g} + {rep['omega']:.3g}; dense residuals {Rr:.6g} / {Rc:.6g}")
    # fp32 potentials: each row's mass carries ~1e-5 max(eps, |f|)/eps relative error
    fl = 1e-5 * max(1.0, float(f.abs().max()) / eps)
    assert max(Rr, Rc) <= R_A + rep["omega"] + fl


@pytest.mark.parametrize("B,d", [(256, 3), (128, 2), (128, 1)])
def test_multiscale_certificate_other_blocks_and_dimensions(sk, B, d):
    """The certified solve with 256-point blocks, and on clouds of the
    clustered workload projected to their first d axes: the certificate bounds
    the exact dense residuals of the returned potentials."""
    n, eps = 16384, 1e-3
    c = synth.make(5, n=n, m=n)
    x = np.ascontiguousarray(c.x[:, :d])
    y = np.ascontiguousarray(c.y[:, :d])
    prm = sk.MultiscaleParams(B=B, eps=eps, tol=1e-2)
    _log(f"multiscale n={n} B={B} d={d}")
    with sk.Problem(_t(x), _t(y), _t(c.a), _t(c.b), 1.0) as P:
        f, g, rep = P.solve_multiscale(prm)
        _log(f"  coarse {rep['coarse_iters']} fine {rep['fine_updates']} cells {rep['ncells_x']}x{rep['ncells_y']}")
        _dense_check(sk, P, rep, eps, f, g, prm.tol)


@pytest.mark.parametrize("eps", [1e-3, 1e-4])
def test_multiscale_certificate_holds_at_2e18(sk, eps):
    """n = m = 2^18 of the clustered workload: the stop certificate bounds the
    exact dense residual of the returned potentials."""
    n = 1 << 18
    c = synth.make(5, n=n, m=n)
    prm = sk.MultiscaleParams(B=128, eps=eps, tol=1e-2)
    _log(f"multiscale n={n} eps={eps}")
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        f, g, rep = P.solve_multiscale(prm)
        _log(f"  coarse {rep['coarse_iters']} fine {rep['fine_updates']} in {rep['seconds_total']:.2f} s")
        _dense_check(sk, P, rep, eps, f, g, prm.tol)


@pytest.mark.parametrize("d", [1, 2])
def test_sparse_halfsteps_low_dimensions(sk, d):
    """The sparse kernels at d = 1 and 2 (clustered points projected to the
    first d axes, Morton order of that cloud), shifted loop with residual."""
    n, B, eps = 6000, 128, 1e-3
    c = synth.make(5, n=n, m=n)
    x = np.ascontiguousarray(c.x[:, :d])
    y = np.ascontiguousarray(c.y[:, :d])
    _, px, _, py = oracle.morton_order(x, y)
    x, y, a, b = x[px], y[py], c.a[px], c.b[py]
    rng = np.random.default_rng(11)
    f, g = _near_plan_potentials(n, eps, rng)
    NB = (n + B - 1) // B
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, 1e-3 / NB)
    ptrT, rowT = oracle.screen_transpose(sx, sy, eps, 1.0, 1e-3 / NB)
    with sk.Problem(_t(x), _t(y), _t(a), _t(b), 1.0) as P:
        got_ptr, got_col = P.block_screen(eps, _t(f), _t(g), B, 1e-3 / NB)
        assert np.array_equal(got_ptr.cpu().numpy(), ptr) and np.array_equal(got_col.cpu().numpy(), col)
        fo, r = P.sparse_halfstep_f(eps, _t(g), B, _t(ptr), _t(col.astype(np.int32)), f_prev=_t(f))
        go, _ = P.sparse_halfstep_g(eps, _t(f), B, _t(ptrT), _t(rowT.astype(np.int32)))
    for got, ref, what in ((fo, oracle.sparse_halfstep_f(x, y, b, g, eps, 1.0, ptr, col, B), "f"),
                           (go, oracle.sparse_halfstep_g(x, y, a, f, eps, 1.0, ptrT, rowT, B), "g")):
        got = got.cpu().numpy().astype(np.float64)
        err = np.abs(got - ref) / np.maximum(eps, np.abs(ref))
        assert err.max() <= 1e-5, (what, d, err.max())
    Rr, _ = oracle.sparse_residuals(x, y, a, b, f, g, eps, 1.0, ptr, col, ptrT, rowT, B)
    assert r == pytest.approx(Rr, rel=1e-3)


# ---- tile verification (FlashSinkhorn 2, §3.2: exact B^2-pair mass of each screened tile)

def _kept_flags(ptr, idx, vptr, vidx):
    """Keep flag per candidate from the verified row-major list."""
    keep = np.zeros(len(idx), bool)
    for I in range(len(ptr) - 1):
        kept = set(vidx[vptr[I]:vptr[I + 1]].tolist())
        keep[ptr[I]:ptr[I + 1]] = [int(J) in kept for J in idx[ptr[I]:ptr[I + 1]]]
    return keep


@pytest.mark.parametrize("n,eps", [(16384, 1e-3), (5000, 1e-3), (65536, 1e-4)])
def test_verify_tiles_match_oracle(sk, n, eps):
    """Keep decisions agree with the fp64 oracle except for tiles whose largest
    share is within 1e-3 of the threshold (fp32 sums decide); the two lists are
    exactly the oracle's compaction of the GPU's decisions."""
    x, y, a, b = _sorted_problem(5, n)
    rng = np.random.default_rng(1)
    f, g = _near_plan_potentials(n, eps, rng)
    B = 128
    NB = MB = (n + B - 1) // B
    delta = 1e-3 / NB
    _log(f"verify n={n} eps={eps}")
    with sk.Problem(_t(x), _t(y), _t(a), _t(b), 1.0) as P:
        ptr, idx = P.block_screen(eps, _t(f), _t(g), B, delta)
        vptr, vidx, tptr, tidx = P.verify_tiles(eps, _t(f), _t(g), B, delta, ptr, idx)
    ptr, idx = ptr.cpu().numpy(), idx.cpu().numpy()
    vptr, vidx = vptr.cpu().numpy(), vidx.cpu().numpy()
    tptr, tidx = tptr.cpu().numpy(), tidx.cpu().numpy()
    keep = _kept_flags(ptr, idx, vptr, vidx)
    assert 0 < keep.sum() < len(idx)
    ref = oracle.verify_tiles(x, y, a, b, f, g, eps, 1.0, ptr, idx, B, delta)
    for e in np.nonzero(keep != ref)[0]:
        I = int(np.searchsorted(ptr, e, side="right") - 1)
        s, t = oracle.tile_shares(x, y, a, b, f, g, eps, 1.0, I, int(idx[e]), B)
        top = max(s.max(), t.max())
        assert abs(top / delta - 1.0) < 1e-3, (I, int(idx[e]), top / delta, keep[e], ref[e])
    ptrV, colV, ptrT, rowsT = oracle.compact_tiles(ptr, idx, keep, MB)
    assert np.array_equal(vptr, ptrV) and np.array_equal(vidx, colV)
    assert np.array_equal(tptr, ptrT) and np.array_equal(tidx, rowsT)


def test_verify_tiles_edge_cases(sk):
    n, eps, B = 1000, 1e-3, 128
    x, y, a, b = _sorted_problem(5, n)
    f, g = _near_plan_potentials(n, eps, np.random.default_rng(3))
    NB = (n + B - 1) // B
    with sk.Problem(_t(x), _t(y), _t(a), _t(b), 1.0) as P:
        # no candidates: empty lists
        ptr0 = torch.zeros(NB + 1, dtype=torch.int64, device=DEV)
        idx0 = torch.zeros(0, dtype=torch.int32, device=DEV)
        vptr, vidx, tptr, tidx = P.verify_tiles(eps, _t(f), _t(g), B, 1e-3, ptr0, idx0)
        assert vidx.numel() == 0 and tidx.numel() == 0
        assert int(vptr.abs().sum()) == 0 and int(tptr.abs().sum()) == 0
        # every tile a candidate and a threshold no share reaches: all kept by
        # the fallbacks
        ptr = torch.arange(NB + 1, dtype=torch.int64, device=DEV) * NB
        idx = torch.arange(NB, dtype=torch.int32, device=DEV).repeat(NB)
        vptr, vidx, tptr, tidx = P.verify_tiles(eps, _t(f), _t(g), B, 1e30, ptr, idx)
        assert torch.equal(vptr, ptr) and torch.equal(vidx, idx)
        # B other than 128, a list that does not start at 0, an index out of range
        with pytest.raises(sk.SinkhornError, match="B = 128") as e:
            P.verify_tiles(eps, _t(f), _t(g), 256, 1e-3, ptr[: (n + 255) // 256 + 1], idx)
        assert e.value.code == sk.ERR_UNSUPPORTED
        with pytest.raises(sk.SinkhornError, match="start at 0") as e:
            P.verify_tiles(eps, _t(f), _t(g), B, 1e-3, ptr + 1, idx)
        assert e.value.code == sk.ERR_INVALID_ARG
        bad = idx.clone()
        bad[3] = NB
        with pytest.raises(sk.SinkhornError, match="out-of-range") as e:
            P.verify_tiles(eps, _t(f), _t(g), B, 1e-3, ptr, bad)
        assert e.value.code == sk.ERR_INVALID_ARG


def test_multiscale_verified_fixed_budget_matches_the_oracle(sk):
    """The fixed-budget solve with tile verification: same cell and iteration
    counts, kept-tile count within fp32 borderline flips, potentials within
    1e-3 eps of the oracle's verified run."""
    path = os.path.join(GOLDEN, "fs2_w5_n16384_fixed_verify.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing {path}: run tests/golden/make_solve_refs.py w5_n16384_fixed_verify")
    ref = dict(np.load(path))
    n = int(ref["n"])
    c = synth.make(5, n=n, m=n)
    eps = float(ref["eps"])
    prm = sk.MultiscaleParams(B=int(ref["B"]), eps=eps, tol=float(ref["tol"]), coarse_tol=float(ref["coarse_tol"]),
                              coarse_max=int(ref["coarse_max"]), stall_window=int(ref["stall_window"]),
                              max_fine=int(ref["max_fine"]), verify=True)
    _log(f"multiscale verified fixed budget n={n}")
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        f, g, rep = P.solve_multiscale(prm)
    assert rep["status"] == sk.NOT_CONVERGED and rep["certified"] == 0
    assert rep["ncells_x"] == int(ref["ncells_x"]) and rep["ncells_y"] == int(ref["ncells_y"])
    assert rep["coarse_iters"] == int(ref["coarse_iters"])
    assert rep["fine_updates"] == int(ref["fine_updates"]) == prm.max_fine
    cands, tiles = int(ref["candidates"][-1]), int(ref["tiles"][-1])
    assert abs(rep["last_candidates"] - cands) <= max(2, cands // 1000), (rep["last_candidates"], cands)
    assert abs(rep["last_tiles"] - tiles) <= max(2, tiles // 200), (rep["last_tiles"], tiles)
    assert rep["last_tiles"] < rep["last_candidates"]
    _gauge_close(f, g, ref["f"], ref["g"], 1e-3 * eps)
    assert rep["R_A_row"] == pytest.approx(float(ref["R_A_row"]), rel=1e-2)


def test_verify_tiles_full_size_sampled(sk):
    """2^24 points, B = 128, every screened tile verified in one launch (more
    tiles than one wave per tile could address); sampled candidates checked
    against the oracle's exact shares: a tile clearly above the threshold is
    kept, a tile clearly below is dropped unless its row or column block
    fallback keeps all of that block's candidates."""
    c = synth.make(5)
    cx, px, cy, py = _gpu_morton(sk, c.x, c.y)
    x, y, a, b = c.x[px], c.y[py], c.a[px], c.b[py]
    eps = 1e-4
    rng = np.random.default_rng(4)
    f, g = _near_plan_potentials(c.n, eps, rng)
    B = 128
    NB = c.n // B
    delta = 1e-3 / NB
    _log("verify full size")
    with sk.Problem(_t(x), _t(y), _t(a), _t(b), 1.0) as P:
        ptr, idx = P.block_screen(eps, _t(f), _t(g), B, delta)
        vptr, vidx, tptr, tidx = P.verify_tiles(eps, _t(f), _t(g), B, delta, ptr, idx)
    nnz = int(idx.shape[0])
    _log(f"  {nnz} candidates, {int(vidx.shape[0])} kept")
    assert nnz > (1 << 22)  # more tiles than one pass of the kernel's grid: the stride loop runs
    ptr, idx = ptr.cpu().numpy(), idx.cpu().numpy()
    vptr, vidx = vptr.cpu().numpy(), vidx.cpu().numpy()
    assert np.array_equal(np.diff(tptr.cpu().numpy()).sum(), len(vidx))
    checked = 0
    for e in np.sort(rng.choice(nnz, 64, replace=False)):
        I = int(np.searchsorted(ptr, e, side="right") - 1)
        J = int(idx[e])
        kept_row = vidx[vptr[I]:vptr[I + 1]]
        kept = bool(np.any(kept_row == J))
        s, t = oracle.tile_shares(x, y, a, b, f, g, eps, 1.0, I, J, B)
        top = max(s.max(), t.max()) / delta
        if abs(top - 1.0) < 1e-3:
            continue
        checked += 1
        if top > 1.0:
            assert kept, (I, J, top)
        elif kept:
            row_all = len(kept_row) == ptr[I + 1] - ptr[I]
            col_all = np.count_nonzero(vidx == J) == np.count_nonzero(idx == J)
            assert row_all or col_all, (I, J, top)
    assert checked >= 48


# ---- sampled residual checks and the adaptive coarse-to-fine switch (FlashSinkhorn 2, §3.1, §B.2)

from oracle.fs2 import sample_indices as _ref_sample_indices  # noqa: E402
from oracle.fs2 import sampled_residual as _ref_sampled_residual  # noqa: E402


@pytest.mark.parametrize("count,k,seed,stream", [(1000, 1024, 0, 0), (1 << 24, 8192, 11, 1),
                                                  (7, 4099, 2**63 + 5, 3), (1, 5, 1, 0)])
def test_sample_indices_bit_exact(sk, count, k, seed, stream):
    got = sk.sample_indices(count, k, seed, stream).cpu().numpy().astype(np.int64)
    assert np.array_equal(got, _ref_sample_indices(count, k, seed, stream))


@pytest.mark.parametrize("side", [0, 1])
def test_sampled_residual_matches_oracle(sk, side):
    c = synth.make(2, n=3000, m=2500)
    eps = 0.01
    res = oracle.solve(c.x, c.y, c.a, c.b, 1.0, oracle.Schedule(eps, eps, fixed_iters=3))
    # both marginals visibly off (a state right after a g-step has a column
    # residual at the fp32 rounding floor of the half-step, ~1e-7)
    rng = np.random.default_rng(6)
    f = (res.f + rng.normal(0, 0.1 * eps, c.n)).astype(np.float32)
    g = (res.g + rng.normal(0, 0.1 * eps, c.m)).astype(np.float32)
    k, seed = 1024, 5
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        est, se = P.sampled_residual(eps, _t(f), _t(g), side=side, k=k, seed=seed)
    if side == 0:
        ref = _ref_sampled_residual(c.x, c.y, c.a, c.b, f, g, eps, 1.0, _ref_sample_indices(c.n, k, seed, 0))
    else:
        ref = _ref_sampled_residual(c.y, c.x, c.b, c.a, g, f, eps, 1.0, _ref_sample_indices(c.m, k, seed, 1))
    assert est == pytest.approx(ref[0], rel=2e-3) and se == pytest.approx(ref[1], rel=2e-3), (est, se, ref)


def test_multiscale_adaptive_fixed_budget_matches_the_oracle(sk):
    """Adaptive switch with an unreachable tol: both sampled checks run (and
    expand to the larger sample) on the same draws as the oracle, then the
    fixed fine budget; check estimates, counts and potentials agree."""
    path = os.path.join(GOLDEN, "fs2_w5_n16384_adaptive.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing {path}: run tests/golden/make_solve_refs.py w5_n16384_adaptive")
    ref = dict(np.load(path))
    n = int(ref["n"])
    c = synth.make(5, n=n, m=n)
    eps = float(ref["eps"])
    prm = sk.MultiscaleParams(B=int(ref["B"]), eps=eps, tol=float(ref["tol"]), coarse_tol=float(ref["coarse_tol"]),
                              coarse_max=int(ref["coarse_max"]), stall_window=int(ref["stall_window"]),
                              max_fine=int(ref["max_fine"]), adaptive=True, check_every=int(ref["check_every"]),
                              check_samples=int(ref["check_samples"]),
                              check_samples_max=int(ref["check_samples_max"]), sample_seed=int(ref["sample_seed"]))
    _log(f"multiscale adaptive fixed budget n={n}")
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        f, g, rep = P.solve_multiscale(prm)
    assert rep["accepted_by_sample"] == 0 and not bool(ref["accepted_by_sample"])
    assert rep["checks"] == int(ref["checks"]) == 2
    assert rep["coarse_iters"] == int(ref["coarse_iters"])
    assert rep["fine_updates"] == int(ref["fine_updates"]) == prm.max_fine
    er, sr, ec, sc, k = ref["check_history"][-1]
    assert rep["last_check_samples"] == int(k) == prm.check_samples_max
    got = rep["last_check"]
    assert got[0] == pytest.approx(er, rel=1e-3) and got[1] == pytest.approx(sr, rel=1e-2), (got, er, sr)
    assert got[2] == pytest.approx(ec, rel=1e-3, abs=1e-9) and got[3] == pytest.approx(sc, rel=1e-2, abs=1e-9)
    _gauge_close(f, g, ref["f"], ref["g"], 1e-3 * eps)


def test_multiscale_adaptive_accepts_an_exact_lift(sk):
    """Singleton cells (the lift is an ordinary half-step): a lift passes the
    sampled check, no fine update runs, and the exact residual of the returned
    potentials is under tol; the oracle takes the same path."""
    rng = np.random.default_rng(12345)
    n = 512
    x = rng.uniform(0, 1, (n, 2)).astype(np.float32)
    y = rng.uniform(0, 1, (n, 2)).astype(np.float32)
    w = np.full(n, 1.0 / n, np.float32)
    kw = dict(B=128, eps=0.005, tol=1e-2, p_bits=42, coarse_tol=0.0, stall_window=1 << 30,
              coarse_iters_per_stage=2, adaptive=True, check_every=3, check_samples=128,
              check_samples_max=512)
    from oracle.fs2 import FS2Params
    ref = oracle.fs2_solve(x, y, w, w, FS2Params(**kw))
    assert ref.accepted_by_sample
    with sk.Problem(_t(x), _t(y), _t(w), _t(w), 1.0) as P:
        f, g, rep = P.solve_multiscale(sk.MultiscaleParams(**kw))
    assert rep["status"] == sk.OK and rep["accepted_by_sample"] == 1 and rep["fine_updates"] == 0
    assert rep["ncells_x"] == n and rep["ncells_y"] == n
    assert abs(rep["checks"] - ref.checks) <= 1, (rep["checks"], ref.checks)
    R = max(oracle.marginal_residuals(x, y, w, w, f.cpu().numpy(), g.cpu().numpy(), kw["eps"], 1.0))
    assert R < kw["tol"]
    if rep["checks"] == ref.checks:
        _gauge_close(f, g, ref.f, ref.g, 1e-3 * kw["eps"])
