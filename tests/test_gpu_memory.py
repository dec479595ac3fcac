"""Working memory of the library on the device (moscot #846, "fix(sparsify):
materialize transport-matrix rows ...": row extraction must not grow with
n * m * k). The library counts every device allocation it makes
(sinkhorn_device_memory), so these checks are exact: a handle holds O(n + m)
workspace, materializing rows into a caller buffer allocates O(k + m), a solve
allocates nothing further, and no buffer anywhere comes near n * m."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

pytestmark = [pytest.mark.gpu, pytest.mark.memory]

torch = pytest.importorskip("torch")
DEV = "cuda:0"

# per point of either side: coordinates, weights, column terms, potentials and
# the split partials of the dense half-steps (at most 64 splits per row, an
# fp64 maximum and an fp32 sum each)
PER_POINT = 1100


@pytest.fixture(scope="module")
def sk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import log_domain_sinkhorn_amd as m

    return m


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _handle_bytes(sk, c, scale=1.0):
    base, _, _ = sk.device_memory(reset=True)
    P = sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), scale)
    cur, peak, big = sk.device_memory()
    return P, cur - base, peak - base, big


@pytest.mark.parametrize("w,d", [(2, 3), (3, 50)], ids=["valu", "mfma"])
def test_handle_workspace_is_linear_in_the_points(sk, w, d):
    sizes = []
    for n, m in ((6000, 5000), (12000, 10000)):
        c = synth.make(w, n=n, m=m, d=d) if w == 3 else synth.make(w, n=n, m=m)
        P, held, peak, big = _handle_bytes(sk, c)
        _log(f"handle w{w} n={n} m={m}: held {held} B, peak {peak} B, largest {big} B")
        P.close()
        assert held <= PER_POINT * (n + m) + (4 << 20), (held, n, m)
        assert big < n * m * 4 // 16, (big, n, m)
        sizes.append(held)
    assert sizes[1] <= 2.5 * sizes[0], sizes


@pytest.mark.parametrize("w,d", [(2, 3), (3, 50)], ids=["valu", "mfma"])
def test_materialize_rows_allocates_no_plan_sized_buffer(sk, w, d):
    n, m, k, eps = 20000, 24000, 1024, 0.05
    c = synth.make(w, n=n, m=m, d=d) if w == 3 else synth.make(w, n=n, m=m)
    start, _, _ = sk.device_memory()
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        f = torch.zeros(n, device=DEV)
        g = torch.zeros(m, device=DEV)
        rows = torch.arange(k, dtype=torch.int64, device=DEV)
        T = torch.empty((k, m), device=DEV)
        torch.cuda.synchronize()
        base, _, _ = sk.device_memory(reset=True)
        P.materialize_rows(eps, f, g, rows, T=T)
        P.min_row(eps, f, g)
        cur, peak, big = sk.device_memory()
    _log(f"materialize w{w}: extra peak {peak - base} B, largest {big} B (k*m*4 = {k * m * 4} B)")
    assert cur == base
    # row terms, keys and an fp64 column term: O(k + m), nothing of k * m
    assert peak - base <= 16 * (k + m) + 4 * (n + m) + (1 << 20), peak - base
    assert big <= 8 * max(k, m, n) + 4096, big
    assert sk.device_memory()[0] == start  # the handle gave everything back


def test_solve_allocates_nothing_further(sk):
    c = synth.make(2, n=4000, m=3000)
    start, _, _ = sk.device_memory()
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        sched = sk.Schedule(eps_start=1.0, eps_target=1e-2, eps_factor=0.5, iters_per_stage=5, tol=1e-3,
                            max_iters=2000)
        f = torch.zeros(c.n, device=DEV)
        g = torch.zeros(c.m, device=DEV)
        torch.cuda.synchronize()
        base, _, _ = sk.device_memory(reset=True)
        P.solve(sched, f, g)
        cur, peak, big = sk.device_memory()
    _log(f"solve: extra peak {peak - base} B, largest {big} B")
    assert cur == base and peak - base <= 1 << 20
    assert sk.device_memory()[0] == start


def test_multiscale_workspace_stays_far_below_the_plan(sk):
    n = 16384
    c = synth.make(5, n=n, m=n)
    prm = sk.MultiscaleParams(B=128, eps=1e-3, tol=1e-2, max_fine=2)
    start, _, _ = sk.device_memory()
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        torch.cuda.synchronize()
        base, _, _ = sk.device_memory(reset=True)
        P.solve_multiscale(prm)
        cur, peak, big = sk.device_memory()
    _log(f"multiscale n={n}: extra peak {peak - base} B, largest {big} B, kept {cur - base} B "
         f"(n*m*4 = {n * n * 4} B)")
    # the handle keeps the sparse launches' dispatch-order scratch (grown on
    # demand: keys, tile indices and sort storage per row tile)
    assert 0 <= cur - base <= 64 * (n // 128) + 4096, cur - base
    assert sk.device_memory()[0] == start
    # sorted sides, cells, codes, the two tile lists (at most NB^2 entries) and scratch
    assert peak - base <= 2 * PER_POINT * 2 * n + 16 * (n // 128) ** 2 + (8 << 20), peak - base
    assert big < n * n * 4 // 64, big
