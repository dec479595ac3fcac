"""GPU parity of the barycentric projection and the source-coordinate gradient
(FlashSinkhorn 2, §A.2, §A.4) against the fp64 oracle.

Tolerance: each coordinate of T within 1e-5 (1 + |T|) of the oracle (the
weights carry the half-step's fp32 exponent rounding, ~1e-6 relative, into a
weighted mean of coordinates of size ~1); the gradient 2 s a_i (x_i - T_i)
within 2 s a_i times the same bound.
"""
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
DEV = "cuda:0"


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


def _close(T, G, Tr, a, scale, x, what):
    T = T.cpu().numpy().astype(np.float64)
    G = G.cpu().numpy().astype(np.float64)
    tol = 1e-5 * (1.0 + np.abs(Tr))
    err = np.abs(T - Tr)
    assert np.all(err <= tol), (what, float((err / tol).max()))
    Gr = oracle.coordinate_gradient(x, a, Tr, scale)
    gtol = 2.0 * scale * np.asarray(a, np.float64)[:, None] * tol + 1e-30
    gerr = np.abs(G - Gr)
    assert np.all(gerr <= gtol), (what, float((gerr / gtol).max()))


def _potentials(sk, P, eps, iters=6):
    g = torch.zeros(P.m, device=DEV)
    for _ in range(iters):
        f, _ = P.halfstep_f(eps, g)
        g, _ = P.halfstep_g(eps, f)
    f, _ = P.halfstep_f(eps, g)
    return f, g


@pytest.mark.parametrize("hint", [True, False], ids=["shifted", "exact"])
@pytest.mark.parametrize("w,n,m,eps", [(2, 3000, 2500, 1e-3), (1, 1000, 1000, 1e-2), (4, 4096, 4913, 1e-3)])
def test_dense_barycentric_matches_oracle(sk, w, n, m, eps, hint):
    c = synth.make(w, n=n, m=m)
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        f, g = _potentials(sk, P, eps)
        T, G = P.barycentric(eps, g, f_hint=f if hint else None)
    Tr = oracle.barycentric_rows(c.x, c.y, c.b, g.cpu().numpy(), eps, 1.0)
    _close(T, G, Tr, c.a, 1.0, c.x, f"w{w}")


def test_dense_barycentric_full_size_sampled_rows(sk):
    """10^6 x 10^6 (d = 3): 48 sampled rows recomputed by the oracle."""
    c = synth.make(4)
    eps = 1e-3
    _log("barycentric 1e6")
    with sk.Problem(_t(c.x), _t(c.y), None, None, 1.0) as P:
        f, g = _potentials(sk, P, eps, iters=2)
        T, G = P.barycentric(eps, g, f_hint=f)
    rows = np.sort(np.random.default_rng(5).choice(c.n, 48, replace=False))
    Tr = oracle.barycentric_rows(c.x, c.y, c.b, g.cpu().numpy(), eps, 1.0, rows=rows)
    _close(T[rows], G[rows], Tr, c.a[rows], 1.0, c.x[rows], "w4 sampled")


@pytest.mark.parametrize("hint", [True, False], ids=["shifted", "exact"])
@pytest.mark.parametrize("n,B,eps", [(16384, 128, 1e-4), (5000, 256, 1e-3)])
def test_sparse_barycentric_matches_oracle(sk, n, B, eps, hint):
    c = synth.make(5, n=n, m=n)
    _, px, _, py = oracle.morton_order(c.x, c.y)
    x, y, a, b = c.x[px], c.y[py], c.a[px], c.b[py]
    rng = np.random.default_rng(9)
    base = eps * np.log(n) / 2
    f = (base + rng.normal(0, 0.3 * eps, n)).astype(np.float32)
    g = (base + rng.normal(0, 0.3 * eps, n)).astype(np.float32)
    NB = (n + B - 1) // B
    sx = oracle.block_summaries(x, a, f, B)
    sy = oracle.block_summaries(y, b, g, B)
    ptr, col = oracle.screen(sx, sy, eps, 1.0, 1e-3 / NB)
    ptr = ptr.copy()  # one empty row block: its rows average over all columns
    col = np.delete(col, np.s_[ptr[1]:ptr[2]])
    ptr[2:] -= ptr[2] - ptr[1]
    with sk.Problem(_t(x), _t(y), _t(a), _t(b), 1.0) as P:
        fh = oracle.sparse_halfstep_f(x, y, b, g, eps, 1.0, ptr, col, B).astype(np.float32)
        T, G = P.sparse_barycentric(eps, _t(g), B, _t(ptr), _t(col.astype(np.int32)),
                                    f_hint=_t(fh) if hint else None)
    Tr = oracle.sparse_barycentric_rows(x, y, b, g, eps, 1.0, ptr, col, B)
    _close(T, G, Tr, a, 1.0, x, "sparse")


def test_barycentric_errors(sk):
    c = synth.make(3, n=200, m=300)
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        with pytest.raises(sk.SinkhornError) as e:
            P.barycentric(0.05, torch.zeros(300, device=DEV))
        assert e.value.code == sk.ERR_UNSUPPORTED  # d = 50
    c = synth.make(2, n=300, m=300)
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        with pytest.raises(sk.SinkhornError) as e:
            P.barycentric(0.01, torch.zeros(300, device=DEV), want_T=False, want_grad=False)
        assert e.value.code == sk.ERR_INVALID_ARG
