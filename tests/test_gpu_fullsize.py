"""Full-size GPU parity, at the sizes the workloads name, wherever the fp64
oracle can follow:

* 2^24 + 2^24 points of the clustered workload (d = 3, B = 128, eps = 1e-4,
  tol = 1e-2), block-sparse solve: certified (FlashSinkhorn 2, §3.1 and §C.4:
  the certificate bounds the exact residual); the exact dense residuals of
  the returned potentials, one side per test (2.8e14 pairs each, fp64 pair
  arithmetic on the GPU, parity-tested against the oracle elsewhere) under
  the certificate; sampled plan rows within 1e-5 relative of the oracle; the
  row- and column-major tile lists at the returned potentials bit-exact
  against the oracle's screen of all 131072 x 131072 block pairs (§3.2); one
  sparse f-step and one sparse g-step on those lists within 1e-5 max(eps, |f|)
  of the oracle on sampled rows, the longest list's block among them.
* 50000 x 60000, d = 50 (eps = 0.05, cost divided by its mean): the min_row
  threshold (moscot #846, "Behavioural changes") at the solved potentials
  within 1e-5 relative of the oracle's over every row, the oracle's pass
  split over four tests.

The 2^24 solve and the d = 50 solve run once per module; every test below
takes at most about a minute and a half on one MI355X.
"""
import math
import sys
import time
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
import synth

import oracle_pool

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(400)]
torch = pytest.importorskip("torch")
DEV = "cuda:0"
TINY = 2.0 ** -126


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


# ------------------------------------------------------------- 2^24 points
@pytest.fixture(scope="module")
def w5(sk):
    c = synth.make(5)
    prm = sk.MultiscaleParams(B=128, eps=1e-4, tol=1e-2)
    _log(f"multiscale n = m = {c.n}, eps {prm.eps}, tol {prm.tol}")
    P = sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0)
    t = time.time()
    f, g, rep = P.solve_multiscale(prm)
    _log(f"  coarse {rep['coarse_iters']} fine {rep['fine_updates']} tiles {rep['last_tiles']} "
         f"in {time.time() - t:.1f} s")
    yield SimpleNamespace(c=c, P=P, f=f, g=g, rep=rep, prm=prm)
    P.close()


def _certificate(w):
    return max(w.rep["R_A_row"], w.rep["R_A_col"]) + w.rep["omega"]


def _floor(w):
    # a residual of fp32 potentials: each row's mass carries ~1e-5 max(eps, |f|)/eps
    return 1e-5 * max(1.0, float(w.f.abs().max()) / w.prm.eps)


def test_w5_full_size_solve_is_certified(sk, w5):
    assert w5.rep["status"] == sk.OK and w5.rep["certified"] == 1
    assert _certificate(w5) <= w5.prm.tol
    assert torch.isfinite(w5.f).all() and torch.isfinite(w5.g).all()


def test_w5_full_size_dense_row_residual_under_the_certificate(w5):
    t = time.time()
    _, Rr = w5.P.halfstep_f(w5.prm.eps, w5.g, f_prev=w5.f)
    _log(f"  dense row residual {Rr:.6g} vs certificate {_certificate(w5):.6g} ({time.time() - t:.1f} s)")
    assert Rr <= _certificate(w5) + _floor(w5)


def test_w5_full_size_dense_column_residual_under_the_certificate(w5):
    t = time.time()
    _, Rc = w5.P.halfstep_g(w5.prm.eps, w5.f, g_prev=w5.g)
    _log(f"  dense column residual {Rc:.6g} vs certificate {_certificate(w5):.6g} ({time.time() - t:.1f} s)")
    assert Rc <= _certificate(w5) + _floor(w5)


def test_w5_full_size_sampled_plan_rows_match_the_oracle(w5):
    c = w5.c
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(c.n, 8, replace=False))
    T, _ = w5.P.materialize_rows(w5.prm.eps, w5.f, w5.g, _t(rows))
    T = T.cpu().numpy().astype(np.float64)
    ref = oracle.materialize_rows(c.x, c.y, c.a, c.b, w5.f.cpu().numpy(), w5.g.cpu().numpy(),
                                  w5.prm.eps, 1.0, rows)
    err = np.abs(T - ref)
    assert not np.any(err > 1e-5 * ref + TINY), int(np.sum(err > 1e-5 * ref + TINY))
    np.testing.assert_allclose(T.sum(axis=1), ref.sum(axis=1), rtol=1e-5)


@pytest.fixture(scope="module")
def w5s(sk, w5):
    """The clouds in the handle's Morton order, the returned potentials in
    that order, and the GPU's tile lists of both orientations there."""
    c = w5.c
    px = w5.P.morton_sort(0)[1].cpu().numpy().astype(np.int64)
    py = w5.P.morton_sort(1)[1].cpu().numpy().astype(np.int64)
    s = SimpleNamespace(x=c.x[px], y=c.y[py], a=c.a[px], b=c.b[py],
                        f=w5.f.cpu().numpy()[px], g=w5.g.cpu().numpy()[py], eps=w5.prm.eps,
                        B=w5.prm.B)
    s.NB = (c.n + s.B - 1) // s.B
    s.MB = (c.m + s.B - 1) // s.B
    s.delta = w5.prm.delta_scale / max(s.NB, s.MB)
    s.P = sk.Problem(_t(s.x), _t(s.y), _t(s.a), _t(s.b), 1.0)
    t = time.time()
    ptr, idx = s.P.block_screen(s.eps, _t(s.f), _t(s.g), s.B, s.delta)
    ptrT, idxT = s.P.block_screen(s.eps, _t(s.f), _t(s.g), s.B, s.delta, transpose=True)
    s.dev = (ptr, idx, ptrT, idxT)
    s.ptr, s.idx = ptr.cpu().numpy(), idx.cpu().numpy()
    s.ptrT, s.idxT = ptrT.cpu().numpy(), idxT.cpu().numpy()
    _log(f"  screens: {len(s.idx)} / {len(s.idxT)} tiles, longest lists {np.diff(s.ptr).max()} / "
         f"{np.diff(s.ptrT).max()} ({time.time() - t:.1f} s)")
    t = time.time()
    s.sx = oracle.block_summaries(s.x, s.a, s.f, s.B)
    s.sy = oracle.block_summaries(s.y, s.b, s.g, s.B)
    _log(f"  oracle block summaries ({time.time() - t:.1f} s)")
    yield s
    s.P.close()


def _lists_bit_exact(s, sa, sb, ptr, idx, what):
    t = time.time()
    ref = oracle_pool.screen_digests(sa, sb, s.eps, 1.0, s.delta)
    _log(f"  oracle screen {what}: {sum(int(r[2].sum()) for r in ref)} tiles "
         f"({time.time() - t:.1f} s, {oracle_pool.workers()} processes)")
    assert ptr[-1] == len(idx) and ptr[0] == 0
    for lo, hi, counts, h in ref:
        got_counts, got_h = oracle_pool.digest(ptr, idx, lo, hi)
        if np.array_equal(got_counts, counts) and got_h == h:
            continue
        # name the first differing block of the range
        rp, rc = oracle.screen(sa, sb, s.eps, 1.0, s.delta, row_blocks=range(lo, hi))
        for k, I in enumerate(range(lo, hi)):
            mine = idx[ptr[I]:ptr[I + 1]]
            theirs = rc[rp[k]:rp[k + 1]]
            assert np.array_equal(mine, theirs), f"{what}: block {I}: {len(mine)} vs {len(theirs)} tiles"
        raise AssertionError(f"{what}: range [{lo}, {hi}) differs")


def test_w5_full_size_row_major_tile_list_bit_exact(w5s):
    _lists_bit_exact(w5s, w5s.sx, w5s.sy, w5s.ptr, w5s.idx, "row-major")


def test_w5_full_size_column_major_tile_list_bit_exact(w5s):
    _lists_bit_exact(w5s, w5s.sy, w5s.sx, w5s.ptrT, w5s.idxT, "column-major")


def _sampled_blocks(ptr, nb, rng):
    counts = np.diff(ptr)
    blocks = {int(np.argmax(counts)): 16, nb - 1: 2}
    empty = np.nonzero(counts == 0)[0]
    if empty.size:
        blocks.setdefault(int(empty[0]), 2)
    for I in rng.choice(nb, 6, replace=False):
        blocks.setdefault(int(I), 2)
    return blocks


def _sparse_rows_match(s, outs, P, Q, wq, pot, ptr, idx, seed, what):
    """Each output's entry i against the oracle's sparse half-step of row i
    alone (its block's list; all columns for an empty list), within
    1e-5 max(eps, |f|)."""
    rng = np.random.default_rng(seed)
    nb = len(ptr) - 1
    worst = {name: 0.0 for name in outs}
    t = time.time()
    for I, k in sorted(_sampled_blocks(ptr, nb, rng).items()):
        lo, hi = I * s.B, min(len(P), (I + 1) * s.B)
        sub = idx[ptr[I]:ptr[I + 1]]
        for i in np.sort(rng.choice(np.arange(lo, hi), min(k, hi - lo), replace=False)):
            ref = oracle.sparse_halfstep_f(P[i:i + 1], Q, wq, pot, s.eps, 1.0,
                                           np.array([0, len(sub)], np.int64), sub, s.B)[0]
            for name, out in outs.items():
                err = abs(float(out[i]) - ref)
                worst[name] = max(worst[name], err / max(s.eps, abs(ref)))
                assert err <= 1e-5 * max(s.eps, abs(ref)), (what, name, I, int(i), float(out[i]), ref,
                                                            len(sub))
    _log(f"  sparse {what}: worst error {worst} of max(eps, |ref|) ({time.time() - t:.1f} s)")


def test_w5_full_size_sparse_f_step_on_sampled_rows(w5s):
    """Both loops: the shifted one (previous potentials given, as in the fine
    updates) and the exact two-pass one (none given)."""
    ptr, idx, _, _ = w5s.dev
    g = _t(w5s.g)
    shifted, _ = w5s.P.sparse_halfstep_f(w5s.eps, g, w5s.B, ptr, idx, f_prev=_t(w5s.f))
    exact, _ = w5s.P.sparse_halfstep_f(w5s.eps, g, w5s.B, ptr, idx)
    outs = {"shifted": shifted.cpu().numpy(), "exact": exact.cpu().numpy()}
    _sparse_rows_match(w5s, outs, w5s.x, w5s.y, w5s.b, w5s.g, w5s.ptr, w5s.idx, 31, "f-step")


def test_w5_full_size_sparse_g_step_on_sampled_columns(w5s):
    _, _, ptrT, idxT = w5s.dev
    f = _t(w5s.f)
    shifted, _ = w5s.P.sparse_halfstep_g(w5s.eps, f, w5s.B, ptrT, idxT, g_prev=_t(w5s.g))
    exact, _ = w5s.P.sparse_halfstep_g(w5s.eps, f, w5s.B, ptrT, idxT)
    outs = {"shifted": shifted.cpu().numpy(), "exact": exact.cpu().numpy()}
    _sparse_rows_match(w5s, outs, w5s.y, w5s.x, w5s.a, w5s.f, w5s.ptrT, w5s.idxT, 32, "g-step")


# ------------------------------------------------- 50000 x 60000, d = 50
W3_PARTS = 4


@pytest.fixture(scope="module")
def w3(sk):
    c = synth.make(3)
    eps = 0.05
    scale = 1.0 / sk.mean_sqeuclid(_t(c.x), _t(c.y))
    _log(f"solve n = {c.n}, m = {c.m}, d = {c.x.shape[1]}, eps {eps}")
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), scale) as P:
        f, g, rep = P.solve(sk.Schedule(eps, eps, tol=1e-3, max_iters=5000))
        assert rep["status"] == sk.OK
        t = time.time()
        mr = P.min_row(eps, f, g)
        _log(f"  {rep['iters']} iterations, R {rep['row_l1']:.3g}; min_row {mr:.9g} "
             f"({time.time() - t:.2f} s)")
    return SimpleNamespace(c=c, eps=eps, scale=scale, f=f.cpu().numpy(), g=g.cpu().numpy(),
                           min_row=float(mr), parts={})


@pytest.mark.parametrize("part", range(W3_PARTS))
def test_w3_full_size_min_row_oracle_part(w3, part):
    """The oracle's min over max_j T_ij for a quarter of the rows."""
    c = w3.c
    lo = part * c.n // W3_PARTS
    hi = (part + 1) * c.n // W3_PARTS
    t = time.time()
    w3.parts[part] = oracle.min_row(c.x[lo:hi], c.y, c.a[lo:hi], c.b, w3.f[lo:hi], w3.g, w3.eps,
                                    w3.scale)
    _log(f"  oracle min_row rows [{lo}, {hi}): {w3.parts[part]:.9g} ({time.time() - t:.1f} s)")
    assert math.isfinite(w3.parts[part]) and w3.parts[part] > 0.0


def test_w3_full_size_min_row_matches_the_oracle(w3):
    assert sorted(w3.parts) == list(range(W3_PARTS))
    ref = min(w3.parts.values())
    assert abs(w3.min_row - ref) <= 1e-5 * ref + TINY, (w3.min_row, ref)
