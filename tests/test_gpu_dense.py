"""GPU parity of the dense online half-steps, the residual and the annealed
solve against the fp64 oracle (same seeded inputs on both sides).

Tolerances (stated with the workloads): one half-step from identical
potentials within 1e-5 * max(eps, |f|) per entry; final potentials within
1e-3 * eps after the same number of iterations.
"""
import math
import os
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _skip_without_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def sk():
    _skip_without_gpu()
    import log_domain_sinkhorn_amd as sk

    return sk


DEV = "cuda:0"


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _problem(sk, c, scale=1.0, uniform=False):
    return sk.Problem(_t(c.x), _t(c.y), None if uniform else _t(c.a), None if uniform else _t(c.b), scale)


def _assert_halfstep(got, ref, eps, what):
    err = np.abs(got.astype(np.float64) - ref) / np.maximum(eps, np.abs(ref))
    worst = int(np.argmax(err))
    assert err.max() <= 1e-5, f"{what}: max rel err {err.max():.3e} at {worst} (got {got[worst]}, ref {ref[worst]})"


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.parametrize(
    "workload,n,m,eps_list",
    [
        (1, None, None, [0.01, 1.0]),
        (2, None, None, [1e-3, 0.125]),
        (2, 1, 1, [1e-2]),
        (2, 37, 1029, [1e-3]),
        (2, 1029, 37, [1e-3]),
        (1, 3001, 517, [1e-2]),
        (4, 4096, 4096, [1e-4, 1e-2]),
    ],
)
def test_single_halfsteps_match_oracle(sk, workload, n, m, eps_list):
    c = synth.make(workload, n=n, m=m)
    _log(f"halfstep parity workload={workload} n={c.n} m={c.m}")
    rng = np.random.default_rng(100 + workload)
    with _problem(sk, c) as P:
        for eps in eps_list:
            g0 = (rng.normal(0, 1, c.m) * eps).astype(np.float32)
            f, _ = P.halfstep_f(eps, _t(g0))
            f_ref = oracle.halfstep_f(c.x, c.y, c.b, g0, eps, 1.0)
            _assert_halfstep(f.cpu().numpy(), f_ref, eps, f"f-step eps={eps}")
            f32 = f_ref.astype(np.float32)
            g, _ = P.halfstep_g(eps, _t(f32))
            g_ref = oracle.halfstep_g(c.x, c.y, c.a, f32, eps, 1.0)
            _assert_halfstep(g.cpu().numpy(), g_ref, eps, f"g-step eps={eps}")


def test_full_size_sampled_rows_workload4(sk):
    """n = m = 10^6 at eps = 1e-4: every row on the GPU, 256 sampled rows and
    columns recomputed by the oracle one by one."""
    c = synth.make(4)
    eps = 1e-4
    rng = np.random.default_rng(44)
    g0 = (rng.normal(0, 1, c.m) * eps).astype(np.float32)
    _log("workload 4 full-size halfstep")
    with _problem(sk, c, uniform=True) as P:
        f, _ = P.halfstep_f(eps, _t(g0))
        f = f.cpu().numpy()
        rows = rng.choice(c.n, 256, replace=False)
        f_ref = oracle.halfstep_f(c.x, c.y, c.b, g0, eps, 1.0, rows=rows)
        _assert_halfstep(f[rows], f_ref, eps, "f-step sampled rows")
        g, _ = P.halfstep_g(eps, _t(f))
        g = g.cpu().numpy()
        cols = rng.choice(c.m, 256, replace=False)
        g_ref = oracle.halfstep_g(c.x, c.y, c.a, f, eps, 1.0, cols=cols)
        _assert_halfstep(g[cols], g_ref, eps, "g-step sampled cols")


def test_massless_points_and_all_massless_side(sk):
    c = synth.make(2, n=300, m=400)
    b = c.b.copy()
    b[::3] = 0.0
    b = (b / b.astype(np.float64).sum()).astype(np.float32)
    a = c.a.copy()
    a[:50] = 0.0
    a = (a / a.astype(np.float64).sum()).astype(np.float32)
    eps = 1e-2
    with sk.Problem(_t(c.x), _t(c.y), _t(a), _t(b), 1.0) as P:
        g0 = np.zeros(c.m, np.float32)
        f, _ = P.halfstep_f(eps, _t(g0))
        _assert_halfstep(f.cpu().numpy(), oracle.halfstep_f(c.x, c.y, b, g0, eps, 1.0), eps, "f with b_j = 0")
        f32 = f.cpu().numpy()
        g, _ = P.halfstep_g(eps, _t(f32))
        _assert_halfstep(g.cpu().numpy(), oracle.halfstep_g(c.x, c.y, a, f32, eps, 1.0), eps, "g with a_i = 0")
    # every exponent -C/eps overflows to -inf: an all -inf row, so f = +inf.
    # The fp64 pair arithmetic overflows where the fp64 oracle does
    # (200 log2(e) / 1e-307 > DBL_MAX); the fp32 loop where its fp32
    # exponent does (eps = 1e-38; its log2(e) / eps must stay below FLT_MAX)
    x = np.zeros((3, 2), np.float32)
    y = np.full((2, 2), 10.0, np.float32)  # |x - y|^2 = 200
    assert np.isinf(oracle.halfstep_f(x, y, np.full(2, 0.5), np.zeros(2), 1e-307, 1.0)).all()
    for flags, tiny in ((0, 1e-307), (sk.FLAG_FP32_PAIRS, 1e-38)):
        with sk.Problem(_t(x), _t(y), None, None, 1.0, flags=flags) as P:
            out = torch.empty(3, device=DEV)
            prev = torch.zeros(3, device=DEV)
            with pytest.raises(sk.SinkhornError) as ei:
                P.halfstep_f(tiny, _t(np.zeros(2, np.float32)), out=out, f_prev=prev)
            assert ei.value.code == sk.ERR_NONFINITE
            assert torch.isinf(out).all(), (flags, out)


def test_init_errors(sk):
    c = synth.make(1, n=10, m=12)
    with pytest.raises(sk.SinkhornError) as ei:
        sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b * 2), 1.0)
    assert ei.value.code == sk.ERR_MASS
    xb = c.x.copy()
    xb[3, 1] = np.nan
    with pytest.raises(sk.SinkhornError) as ei:
        sk.Problem(_t(xb), _t(c.y), _t(c.a), _t(c.b), 1.0)
    assert ei.value.code == sk.ERR_NONFINITE


def test_problem_info_reports_the_handles_sizes(sk):
    c = synth.make(3, n=37, m=53, d=50)
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 0.125) as P:
        assert P.info() == (37, 53, 50, 0.125)
        # every output is optional
        assert sk.lib().sinkhorn_problem_info(P._h, None, None, None, None) == sk.OK


def test_measurement_hook_counts_each_kind(sk):
    """A half-step with a previous potential runs the shifted loop (dense
    kind), one without runs the exact loop (its own kind); each launch is
    counted once with its n*m pairs and a positive kernel time."""
    c = synth.make(2, n=3000, m=2000)
    eps = 0.01
    with _problem(sk, c) as P:
        g = torch.zeros(c.m, device=DEV)
        f, _ = P.halfstep_f(eps, g)
        for kinds, prev, want in ((sk.PROF_DENSE, True, 1), (sk.PROF_DENSE, False, 0),
                                  (sk.PROF_DENSE_EXACT, False, 1), (sk.PROF_DENSE_EXACT, True, 0)):
            P.profile_enable(kinds)
            P.halfstep_f(eps, g, f_prev=f if prev else None)
            ms, launches, pairs = P.profile_read()
            P.profile_enable(0)
            assert launches == want, (kinds, prev, launches)
            assert pairs == pytest.approx(want * c.n * c.m)
            assert (ms > 0.0) == (want > 0)


def test_fused_row_residual_matches_explicit_plan(sk):
    c = synth.make(2, n=1500, m=1300)
    eps = 5e-3
    rng = np.random.default_rng(3)
    f0 = (rng.normal(0, 1, c.n) * eps).astype(np.float32)
    g0 = (rng.normal(0, 1, c.m) * eps).astype(np.float32)
    with _problem(sk, c) as P:
        _, r = P.halfstep_f(eps, _t(g0), f_prev=_t(f0))
        _, cr = P.halfstep_g(eps, _t(f0), g_prev=_t(g0))
        R_row, R_col = oracle.marginal_residuals(c.x, c.y, c.a, c.b, f0, g0, eps, 1.0)
        # error of the half-step (1e-5 max(eps,|f|)) propagated through exp(./eps)
        f_ref = oracle.halfstep_f(c.x, c.y, c.b, g0, eps, 1.0)
        bound = (c.a * np.exp((f0 - f_ref) / eps) * 1e-5 * np.maximum(eps, np.abs(f_ref)) / eps).sum()
        assert abs(r - R_row) <= bound + 1e-12, (r, R_row, bound)
        g_ref = oracle.halfstep_g(c.x, c.y, c.a, f0, eps, 1.0)
        bound = (c.b * np.exp((g0 - g_ref) / eps) * 1e-5 * np.maximum(eps, np.abs(g_ref)) / eps).sum()
        assert abs(cr - R_col) <= bound + 1e-12, (cr, R_col, bound)
        rr, cc = P.marginal_residual(eps, _t(f0), _t(g0))
        assert rr == r and cc == cr  # the same kernels, deterministic


def test_mean_sqeuclid(sk):
    c = synth.make(3, n=3000, m=2000)
    got = sk.mean_sqeuclid(_t(c.x), _t(c.y))
    assert got == pytest.approx(oracle.mean_sqeuclid(c.x, c.y), rel=1e-10)


def test_bit_reproducible(sk):
    c = synth.make(2, n=5000, m=7000)
    g0 = np.zeros(c.m, np.float32)
    with _problem(sk, c) as P:
        f1, _ = P.halfstep_f(1e-3, _t(g0))
        f2, _ = P.halfstep_f(1e-3, _t(g0))
        assert torch.equal(f1, f2)


GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    path = os.path.join(GOLDEN, f"solve_{name}.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing {path}: run tests/golden/make_solve_refs.py")
    return dict(np.load(path))


def _schedule(sk, ref, **over):
    kw = dict(eps_start=float(ref["eps_start"]), eps_target=float(ref["eps_target"]),
              eps_factor=float(ref["eps_factor"]), iters_per_stage=int(ref["iters_per_stage"]),
              fixed_iters=int(ref["fixed_iters"]), tol=float(ref["tol"]), max_iters=int(ref["max_iters"]))
    kw.update(over)
    return sk.Schedule(**kw)


def _golden_problem(sk, ref):
    c = synth.make(int(ref["workload"]), n=int(ref["n"]), m=int(ref["m"]))
    return c, sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), float(ref["scale"]))


def _record(name, **vals):
    """Append the measured figures of a parity case to the file named by
    SINKHORN_PARITY_LOG (one JSON line), when that variable is set."""
    path = os.environ.get("SINKHORN_PARITY_LOG")
    if path:
        import json

        with open(path, "a") as fh:
            fh.write(json.dumps({"case": name, **vals}) + "\n")


def _potentials_close(f, g, ref, eps, name):
    """Raw potentials within 1e-3 eps of the oracle's after the same iteration
    count (no gauge fixing: both sides run the same iteration from f = g = 0,
    so the free shift (f + c, g - c) of FlashSinkhorn 2, §A.3 is the same on
    both)."""
    f = f.cpu().numpy().astype(np.float64)
    g = g.cpu().numpy().astype(np.float64)
    df = float(np.abs(f - ref["f"]).max())
    dg = float(np.abs(g - ref["g"]).max())
    _log(f"{name}: max |f - f_ref| = {df:.3e}, max |g - g_ref| = {dg:.3e} ({max(df, dg) / eps:.2e} eps)")
    _record(name, eps=eps, iters=int(ref["iters"]), df=df, dg=dg, drift_over_eps=max(df, dg) / eps)
    assert df <= 1e-3 * eps and dg <= 1e-3 * eps, (df, dg, 1e-3 * eps)


SOLVE_GOLDENS = ["w1_full_fixed200", "w2_n1000_tol", "w4_n1000_tol", "w3_n1500_tol"]
# full-size goldens (hours of fp64 numpy to write)
for _name in ("w2_full_tol", "w3_full_fixed10"):
    if os.path.exists(os.path.join(GOLDEN, f"solve_{_name}.npz")):
        SOLVE_GOLDENS.append(_name)


@pytest.mark.parametrize("name", SOLVE_GOLDENS)
def test_solve_same_iteration_count_gives_same_potentials(sk, name):
    """Run exactly the oracle's iteration count, then compare the potentials
    (within 1e-3 eps) and the residual the solve reports."""
    ref = _golden(name)
    eps = float(ref["eps_target"])
    _log(f"solve parity {name} ({int(ref['iters'])} iterations)")
    c, P = _golden_problem(sk, ref)
    with P:
        f, g, rep = P.solve(_schedule(sk, ref, fixed_iters=int(ref["final_iters"])))
        assert rep["status"] == sk.OK and rep["iters"] == int(ref["iters"])
        _potentials_close(f, g, ref, eps, name)
        # a residual computed from fp32 potentials carries the half-step
        # tolerance through exp(./eps): sum_i a_i 1e-5 max(eps, |f_i|) / eps
        floor = float((c.a * 1e-5 * np.maximum(eps, np.abs(ref["f"])) / eps).sum())
        assert abs(rep["row_l1"] - float(ref["R_row"])) <= 2e-2 * float(ref["R_row"]) + floor


@pytest.mark.parametrize("name", [n for n in SOLVE_GOLDENS if n.endswith("_tol")])
def test_solve_stops_at_the_oracles_iteration(sk, name):
    """Tolerance mode: the residual test fires at the oracle's iteration (one
    iteration of slack, since both residuals sit within rounding of tol there);
    on the same iteration the potentials agree within 1e-3 eps."""
    ref = _golden(name)
    c, P = _golden_problem(sk, ref)
    with P:
        f, g, rep = P.solve(_schedule(sk, ref))
    assert rep["status"] == sk.OK and rep["converged"] == 1
    assert abs(rep["iters"] - int(ref["iters"])) <= 1, (rep["iters"], int(ref["iters"]))
    assert rep["row_l1"] <= float(ref["tol"])
    _record(name + ":tol", iters=int(rep["iters"]), oracle_iters=int(ref["iters"]), row_l1=rep["row_l1"])
    if rep["iters"] == int(ref["iters"]):
        _potentials_close(f, g, ref, float(ref["eps_target"]), name + ":tol")


def test_small_eps_long_solve_matches_at_plan_level(sk):
    """eps = 1e-4 after 2229 iterations (|f| up to 0.045 = 450 eps): besides
    the potentials (checked above within 1e-3 eps), the oracle's exact marginal
    residuals of the GPU potentials stay at the tolerance and the transport
    cost <pi, C> moves no more than the potentials allow: every plan entry
    changes by a factor within exp(+-(max|df| + max|dg|)/eps), so the cost
    by at most that factor minus one (relative)."""
    ref = _golden("w4_n1000_tol")
    eps = float(ref["eps_target"])
    c, P = _golden_problem(sk, ref)
    with P:
        f, g, rep = P.solve(_schedule(sk, ref, fixed_iters=int(ref["final_iters"])))
    assert rep["iters"] == int(ref["iters"])
    f = f.cpu().numpy().astype(np.float64)
    g = g.cpu().numpy().astype(np.float64)
    R_row, R_col = oracle.marginal_residuals(c.x, c.y, c.a, c.b, f, g, eps, 1.0)
    assert max(R_row, R_col) <= 1.01 * float(ref["tol"]), (R_row, R_col)
    C = oracle.cost_rows(c.x, c.y, 1.0)
    cost = float((oracle.plan_rows(c.x, c.y, c.a, c.b, f, g, eps, 1.0) * C).sum())
    cost_ref = float((oracle.plan_rows(c.x, c.y, c.a, c.b, ref["f"], ref["g"], eps, 1.0) * C).sum())
    shift = (np.abs(f - ref["f"]).max() + np.abs(g - ref["g"]).max()) / eps
    assert shift <= 2e-3, shift
    assert abs(cost - cost_ref) <= math.expm1(shift) * cost_ref, (cost, cost_ref, shift)


def test_solve_not_converged_returns_valid_potentials(sk):
    c = synth.make(2, n=800, m=900)
    with _problem(sk, c) as P:
        f, g, rep = P.solve(sk.Schedule(1e-3, 1e-3, tol=1e-12, max_iters=5))
    assert rep["status"] == sk.NOT_CONVERGED and rep["final_iters"] == 5
    ref = oracle.solve(c.x, c.y, c.a, c.b, 1.0, oracle.Schedule(1e-3, 1e-3, fixed_iters=5))
    assert np.abs(f.cpu().numpy() - ref.f).max() <= 1e-3 * 1e-3


@pytest.mark.parametrize("offset", [0.0, 300.0, -300.0, "mixed"])
def test_shifted_pair_loop_matches_oracle_for_any_shift_estimate(sk, offset):
    """With a previous potential the half-step runs the shifted pair loop,
    whose per-row shift comes from that potential. A good estimate, one far
    too low (chunk sums overflow: exact redo of the chunk), one far too high
    (row sums underflow: exact recompute of the tile) and a mixture must all
    give the oracle's potentials."""
    c = synth.make(2, n=3000, m=2500)
    eps = 1e-3
    rng = np.random.default_rng(21)
    g0 = (rng.normal(0, 1, c.m) * eps).astype(np.float32)
    f_ref = oracle.halfstep_f(c.x, c.y, c.b, g0, eps, 1.0)
    if offset == "mixed":
        prev = f_ref + rng.choice([-300.0, 0.0, 300.0], c.n) * eps
    else:
        prev = f_ref + offset * eps
    with _problem(sk, c) as P:
        f, _ = P.halfstep_f(eps, _t(g0), f_prev=_t(prev.astype(np.float32)))
        _assert_halfstep(f.cpu().numpy(), f_ref, eps, f"shifted f-step offset={offset}")
        g_ref = oracle.halfstep_g(c.x, c.y, c.a, f_ref.astype(np.float32), eps, 1.0)
        gprev = (g_ref - (300.0 if offset == 300.0 else 0.0) * eps).astype(np.float32)
        g, _ = P.halfstep_g(eps, _t(f_ref.astype(np.float32)), g_prev=_t(gprev))
        _assert_halfstep(g.cpu().numpy(), g_ref, eps, f"shifted g-step offset={offset}")


def test_split_form_column_terms_beyond_two_to_the_22(sk):
    """Potentials near 3 at eps = 1e-6 put every column term
    h_j = log2 b_j + g_j log2(e) / eps near 4.3e6, past 2^22, where the split
    takes the fp32 rounding of h_j as its integer part and keeps the rest in
    the weight: the shifted f-step stays within eps of the oracle (the fp32
    output itself rounds to about 0.12 eps at |f| = 3)."""
    c = synth.make(2, n=700, m=900)
    eps = 1e-6
    rng = np.random.default_rng(23)
    g0 = (3.0 + rng.normal(0, 1, c.m) * eps).astype(np.float32)
    h = np.log2(c.b.astype(np.float64)) + g0.astype(np.float64) * (1.0 / math.log(2.0)) / eps
    assert (np.abs(h) > 2.0 ** 22).all()
    f_ref = oracle.halfstep_f(c.x, c.y, c.b, g0, eps, 1.0)
    with _problem(sk, c) as P:
        f, _ = P.halfstep_f(eps, _t(g0), f_prev=_t(f_ref.astype(np.float32)))
    f = f.cpu().numpy().astype(np.float64)
    _assert_halfstep(f, f_ref, eps, "split form, |h| > 2^22")
    assert np.abs(f - f_ref).max() <= eps, np.abs(f - f_ref).max() / eps


def test_shifted_full_size_workload4_sampled_rows(sk):
    c = synth.make(4)
    eps = 1e-4
    rng = np.random.default_rng(45)
    g0 = (rng.normal(0, 1, c.m) * eps).astype(np.float32)
    with _problem(sk, c, uniform=True) as P:
        f0, _ = P.halfstep_f(eps, _t(g0))
        f1, _ = P.halfstep_f(eps, _t(g0), f_prev=f0)  # shifted, good estimate
        assert torch.equal(f0, f1) or float((f0 - f1).abs().max()) <= 1e-5 * max(eps, float(f0.abs().max()))
        rows = rng.choice(c.n, 128, replace=False)
        f_ref = oracle.halfstep_f(c.x, c.y, c.b, g0, eps, 1.0, rows=rows)
        _assert_halfstep(f1.cpu().numpy()[rows], f_ref, eps, "shifted f-step sampled rows")


@pytest.mark.parametrize("d", [1, 4, 5, 8])
@pytest.mark.parametrize("shifted", [False, True], ids=["exact", "shifted"])
def test_halfsteps_in_other_dimensions(sk, d, shifted):
    """The VALU kernels for every d <= 8 (the PCA-like generator in d
    dimensions, cost divided by its mean, ragged sizes)."""
    c = synth.make(3, n=1100, m=1337, d=d)
    scale = 1.0 / oracle.mean_sqeuclid(c.x, c.y)
    eps = 0.02
    rng = np.random.default_rng(40 + d)
    g0 = (rng.normal(0, 1, c.m) * eps).astype(np.float32)
    f_ref = oracle.halfstep_f(c.x, c.y, c.b, g0, eps, scale)
    prev = (f_ref + rng.normal(0, 3 * eps, c.n)).astype(np.float32)  # a rough shift estimate
    _log(f"halfstep d={d} shifted={shifted}")
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), scale) as P:
        f, r = P.halfstep_f(eps, _t(g0), f_prev=_t(prev) if shifted else None)
        _assert_halfstep(f.cpu().numpy(), f_ref, eps, f"f-step d={d}")
        f32 = f_ref.astype(np.float32)
        g, _ = P.halfstep_g(eps, _t(f32))
        _assert_halfstep(g.cpu().numpy(), oracle.halfstep_g(c.x, c.y, c.a, f32, eps, scale), eps, f"g-step d={d}")
        if shifted:  # the fused residual of (prev, g0)
            ref = oracle.row_residual_identity(c.a, prev, f_ref, eps)
            assert r == pytest.approx(ref, rel=1e-3)


def test_both_pair_precisions_match_the_oracle_and_the_report(sk):
    """The default fp64 pair arithmetic (d <= 3) and the fp32 loop selected by
    SINKHORN_FLAG_FP32_PAIRS both give half-steps within 1e-5 max(eps, |f|),
    in exact and shifted mode; the solve report carries the residual history
    (the last checks, the final one the row residual that passed), the
    handle's workspace and no allocation during a dense solve."""
    c = synth.make(2, n=1500, m=1300)
    eps = 1e-3
    rng = np.random.default_rng(9)
    g0 = (rng.normal(0, 1, c.m) * eps).astype(np.float32)
    f_ref = oracle.halfstep_f(c.x, c.y, c.b, g0, eps, 1.0)
    prev = (f_ref + rng.normal(0, 5 * eps, c.n)).astype(np.float32)
    for flags in (0, sk.FLAG_FP32_PAIRS):
        base, _, _ = sk.device_memory(reset=True)
        with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0, flags=flags) as P:
            held, _, _ = sk.device_memory()
            f, _ = P.halfstep_f(eps, _t(g0))
            _assert_halfstep(f.cpu().numpy(), f_ref, eps, f"exact f-step flags={flags}")
            f, r = P.halfstep_f(eps, _t(g0), f_prev=_t(prev))
            _assert_halfstep(f.cpu().numpy(), f_ref, eps, f"shifted f-step flags={flags}")
            assert r == pytest.approx(oracle.row_residual_identity(c.a, prev, f_ref, eps), rel=1e-3)
            _, _, rep = P.solve(sk.Schedule(1.0, eps, tol=1e-3, max_iters=3000), history=8)
        assert rep["status"] == sk.OK and rep["converged"] == 1
        assert rep["workspace_bytes"] == held - base and rep["peak_extra_bytes"] == 0
        assert rep["seconds_per_halfstep"] == pytest.approx(rep["seconds"] / rep["halfsteps"])
        hist = rep["history"]
        assert rep["history_len"] >= len(hist) == min(8, rep["history_len"]) >= 1
        assert hist[-1] == rep["row_l1"] <= 1e-3 and all(h > 1e-3 for h in hist[:-1])
