"""GPU parity of the MFMA half-step (d > 8, cross term on fp32 MFMA over
centred clouds) against the fp64 oracle, on workload-3 style clouds with the
cost scaled by 1 / mean squared distance (a number resolved once)."""
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


def _check(got, ref, eps, what):
    err = np.abs(got.astype(np.float64) - ref) / np.maximum(eps, np.abs(ref))
    k = int(np.argmax(err))
    assert err.max() <= 1e-5, f"{what}: max rel err {err.max():.3e} at {k} (got {got[k]}, ref {ref[k]})"


@pytest.mark.parametrize("n,m,d", [(1500, 1800, 50), (37, 1029, 50), (1029, 37, 50), (700, 900, 9),
                                   (600, 500, 17), (513, 400, 63), (1, 1, 50)])
def test_mfma_halfsteps_match_oracle(sk, n, m, d):
    c = synth.make(3, n=n, m=m, d=d)
    scale = 1.0 / oracle.mean_sqeuclid(c.x, c.y)
    _log(f"mfma halfstep n={n} m={m} d={d} scale={scale:.4g}")
    rng = np.random.default_rng(7)
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), scale) as P:
        for eps in (0.05, 0.5):
            g0 = (rng.normal(0, 1, c.m) * eps).astype(np.float32)
            f, _ = P.halfstep_f(eps, _t(g0))
            f_ref = oracle.halfstep_f(c.x, c.y, c.b, g0, eps, scale)
            _check(f.cpu().numpy(), f_ref, eps, f"f-step eps={eps}")
            f32 = f_ref.astype(np.float32)
            g, _ = P.halfstep_g(eps, _t(f32))
            g_ref = oracle.halfstep_g(c.x, c.y, c.a, f32, eps, scale)
            _check(g.cpu().numpy(), g_ref, eps, f"g-step eps={eps}")


def test_mfma_full_size_sampled_rows(sk):
    c = synth.make(3)
    scale = 1.0 / sk.mean_sqeuclid(_t(c.x), _t(c.y))
    eps = 0.05
    rng = np.random.default_rng(33)
    g0 = (rng.normal(0, 1, c.m) * eps).astype(np.float32)
    _log("mfma full-size 50000 x 60000")
    with sk.Problem(_t(c.x), _t(c.y), None, None, scale) as P:
        f, _ = P.halfstep_f(eps, _t(g0))
        f = f.cpu().numpy()
        rows = rng.choice(c.n, 128, replace=False)
        _check(f[rows], oracle.halfstep_f(c.x, c.y, c.b, g0, eps, scale, rows=rows), eps, "f rows")
        g, _ = P.halfstep_g(eps, _t(f))
        g = g.cpu().numpy()
        cols = rng.choice(c.m, 128, replace=False)
        _check(g[cols], oracle.halfstep_g(c.x, c.y, c.a, f, eps, scale, cols=cols), eps, "g cols")


def test_mfma_residual_and_solve_parity(sk):
    ref = dict(np.load(os.path.join(GOLDEN, "solve_w3_n1500_tol.npz")))
    c = synth.make(3, n=int(ref["n"]), m=int(ref["m"]))
    scale = float(ref["scale"])
    eps = float(ref["eps_target"])
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), scale) as P:
        sched = sk.Schedule(eps, eps, tol=float(ref["tol"]), max_iters=int(ref["max_iters"]))
        f, g, rep = P.solve(sched)
        assert rep["status"] == sk.OK
        assert abs(rep["iters"] - int(ref["iters"])) <= 1, (rep["iters"], int(ref["iters"]))
        sched.fixed_iters = int(ref["final_iters"])
        f, g, rep = P.solve(sched)
        df = np.abs(f.cpu().numpy() - ref["f"]).max()
        dg = np.abs(g.cpu().numpy() - ref["g"]).max()
        assert df <= 1e-3 * eps and dg <= 1e-3 * eps, (df, dg)
        r, cres = P.marginal_residual(eps, f, g)
        R_row, R_col = oracle.marginal_residuals(c.x, c.y, c.a, c.b, f.cpu().numpy(), g.cpu().numpy(), eps, scale)
        fl = float((c.a * 1e-5 * np.maximum(eps, np.abs(ref["f"])) / eps).sum())
        assert abs(r - R_row) <= 1e-2 * R_row + fl and abs(cres - R_col) <= 1e-2 * R_col + fl
