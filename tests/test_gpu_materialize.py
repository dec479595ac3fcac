"""GPU parity of the transport-plan row materializer and the min_row threshold
(moscot #846) against the fp64 oracle.

Tolerance: each entry within 1e-5 relative of the oracle; entries below the
smallest normal fp32 number (2^-126) are compared absolutely at that level,
since fp32 cannot hold them.
"""
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu
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


def _rows_close(T, ref, what):
    err = np.abs(T.astype(np.float64) - ref)
    bad = err > 1e-5 * ref + TINY
    if bad.any():
        r, c = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} entries off, e.g. [{r},{c}] got {T[r, c]} ref {ref[r, c]}")


CASES = [
    # workload, n, m, d, eps, scale rule
    (2, 700, 900, None, 1e-2, "one"),
    (1, 333, 1029, None, 0.01, "one"),
    (3, 1500, 1800, 50, 0.05, "mean"),
    (3, 300, 77, 17, 0.05, "mean"),
]


@pytest.mark.parametrize("w,n,m,d,eps,rule", CASES)
def test_rows_and_row_max_match_oracle(sk, w, n, m, d, eps, rule):
    c = synth.make(w, n=n, m=m, d=d)
    scale = 1.0 if rule == "one" else 1.0 / oracle.mean_sqeuclid(c.x, c.y)
    rng = np.random.default_rng(5)
    g = (rng.normal(0, 1, c.m) * eps).astype(np.float32)
    f = oracle.halfstep_f(c.x, c.y, c.b, g, eps, scale).astype(np.float32)
    rows = np.concatenate([rng.choice(c.n, min(c.n, 37), replace=False), [0, c.n - 1, 0]]).astype(np.int64)
    _log(f"materialize w={w} n={n} m={m} d={c.d} k={len(rows)}")
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), scale) as P:
        rm = torch.empty(len(rows), device=DEV)
        T, _ = P.materialize_rows(eps, _t(f), _t(g), _t(rows), row_max=rm)
        T = T.cpu().numpy()
        ref = oracle.materialize_rows(c.x, c.y, c.a, c.b, f, g, eps, scale, rows)
        _rows_close(T, ref, "rows")
        np.testing.assert_allclose(rm.cpu().numpy(), ref.max(axis=1), rtol=1e-5)
        # right after an f-step every row sums to a_i
        np.testing.assert_allclose(T.astype(np.float64).sum(1), c.a[rows], rtol=2e-5)


@pytest.mark.parametrize("w,n,m,d,eps,rule", CASES)
def test_min_row_matches_oracle_with_massless_rows(sk, w, n, m, d, eps, rule):
    c = synth.make(w, n=n, m=m, d=d)
    a = c.a.copy()
    a[::5] = 0.0  # massless rows take no part in the threshold
    a = (a / a.astype(np.float64).sum() * c.b.astype(np.float64).sum()).astype(np.float32)
    scale = 1.0 if rule == "one" else 1.0 / oracle.mean_sqeuclid(c.x, c.y)
    rng = np.random.default_rng(6)
    g = (rng.normal(0, 1, c.m) * eps).astype(np.float32)
    f = oracle.halfstep_f(c.x, c.y, c.b, g, eps, scale).astype(np.float32)
    with sk.Problem(_t(c.x), _t(c.y), _t(a), _t(c.b), scale) as P:
        got = P.min_row(eps, _t(f), _t(g))
    ref = oracle.min_row(c.x, c.y, a, c.b, f, g, eps, scale)
    assert got == pytest.approx(ref, rel=1e-5)


def test_full_size_d50_batch_of_1024_rows(sk):
    c = synth.make(3)
    scale = 1.0 / sk.mean_sqeuclid(_t(c.x), _t(c.y))
    eps = 0.05
    rng = np.random.default_rng(9)
    f = (rng.normal(0, 1, c.n) * eps).astype(np.float32)
    g = (rng.normal(0, 1, c.m) * eps).astype(np.float32)
    rows = np.sort(rng.choice(c.n, 1024, replace=False)).astype(np.int64)
    _log("materialize 1024 x 60000, d=50")
    with sk.Problem(_t(c.x), _t(c.y), None, None, scale) as P:
        T, _ = P.materialize_rows(eps, _t(f), _t(g), _t(rows))
        T = T.cpu().numpy()
    pick = rng.choice(1024, 12, replace=False)
    ref = oracle.materialize_rows(c.x, c.y, c.a, c.b, f, g, eps, scale, rows[pick])
    _rows_close(T[pick], ref, "sampled rows of the batch")


def test_bad_row_index_is_rejected(sk):
    c = synth.make(1, n=100, m=80)
    with sk.Problem(_t(c.x), _t(c.y), None, None, 1.0) as P:
        z = torch.zeros(100, device=DEV)
        zg = torch.zeros(80, device=DEV)
        with pytest.raises(sk.SinkhornError) as ei:
            P.materialize_rows(0.1, z, zg, _t(np.array([3, 100], np.int64)))
        assert ei.value.code == sk.ERR_INVALID_ARG


@pytest.mark.parametrize("w,n,m,d,eps,rule", CASES)
def test_sparsify_at_min_row_matches_rows_and_oracle(sk, w, n, m, d, eps, rule):
    """moscot #846 thresholding on the device: the CSR holds exactly the
    entries of the GPU's own materialized rows that reach min_row (same
    arithmetic, so bit-exact), every row with mass keeps its largest entry,
    and against the fp64 oracle the kept set agrees wherever an entry is not
    within rounding (2e-5 relative) of the threshold."""
    c = synth.make(w, n=n, m=m, d=d)
    a = c.a.copy()
    a[::7] = 0.0
    a = (a / a.astype(np.float64).sum() * c.b.astype(np.float64).sum()).astype(np.float32)
    scale = 1.0 if rule == "one" else 1.0 / oracle.mean_sqeuclid(c.x, c.y)
    rng = np.random.default_rng(8)
    g = (rng.normal(0, 1, c.m) * eps).astype(np.float32)
    f = oracle.halfstep_f(c.x, c.y, c.b, g, eps, scale).astype(np.float32)
    with sk.Problem(_t(c.x), _t(c.y), _t(a), _t(c.b), scale) as P:
        thr = P.min_row(eps, _t(f), _t(g))
        ptr, col, val = P.sparsify(eps, _t(f), _t(g), thr, batch=64)
        T, _ = P.materialize_rows(eps, _t(f), _t(g), _t(np.arange(c.n, dtype=np.int64)))
        T = T.cpu().numpy()
        # a too-small capacity: the count and row pointers still come back
        with pytest.raises(sk.SinkhornError) as ei:
            P.sparsify(eps, _t(f), _t(g), thr, cap=int(ptr[-1].item()) - 1)
        assert ei.value.code == sk.ERR_CAPACITY
    ptr, col, val = ptr.cpu().numpy(), col.cpu().numpy(), val.cpu().numpy()
    per_row = np.diff(ptr)
    assert np.all(per_row[a == 0] == 0) and np.all(per_row[a > 0] >= 1)
    for i in range(c.n):  # bit-exact against the GPU's own rows
        keep = np.nonzero(T[i] >= thr)[0]
        assert np.array_equal(col[ptr[i]:ptr[i + 1]], keep), i
        assert np.array_equal(val[ptr[i]:ptr[i + 1]], T[i, keep]), i
    ref = oracle.materialize_rows(c.x, c.y, a, c.b, f, g, eps, scale, np.arange(c.n))
    sure = np.abs(ref - thr) > 2e-5 * thr
    assert np.array_equal((T >= thr)[sure], (ref >= thr)[sure])
    kept = T >= thr
    np.testing.assert_allclose(T[kept], ref[kept], rtol=1e-5)
