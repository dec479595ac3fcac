"""The allocation-free materializer (sinkhorn_materialize_rows_noalloc) against
sinkhorn_materialize_rows on the GPU: the same plan rows and row maxima bit
for bit, on two calls in a row with the second smaller (its buffers hold the
first call's values), no device memory allocated by the library during the
calls, and sizes beyond the stated limits refused."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def sk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import log_domain_sinkhorn_amd as sk

    return sk


DEV = "cuda:0"


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _potentials(sk, P, eps, n, m):
    f = torch.zeros(n, dtype=torch.float32, device=DEV)
    g = torch.zeros(m, dtype=torch.float32, device=DEV)
    f, g, _ = P.solve(sk.Schedule(eps, eps, fixed_iters=20), f, g)
    return f, g


def _both(sk, P, eps, f, g, rows, m):
    k = rows.shape[0]
    T0, r0 = P.materialize_rows(eps, f, g, rows, row_max=torch.empty(k, device=DEV))
    T1 = torch.full((k, m), float("nan"), device=DEV)
    r1 = torch.full((k,), float("nan"), device=DEV)
    torch.cuda.synchronize()
    sk.device_memory(reset=True)
    cur0, _, _ = sk.device_memory()
    P.materialize_rows_noalloc(eps, f, g, rows, T1, row_max=r1)
    cur, peak, largest = sk.device_memory()
    assert cur == cur0 and peak == cur0 and largest == 0  # nothing allocated by the call
    assert torch.equal(T0, T1)
    assert torch.equal(r0, r1)
    return T1


@pytest.mark.parametrize("workload,d", [(2, None), (3, 50)], ids=["valu_d3", "mfma_d50"])
def test_noalloc_rows_equal_the_allocating_entry_point(sk, workload, d):
    eps = 1e-2 if workload == 2 else 0.05
    big = synth.make(workload, n=3000, m=2900, **({"d": d} if d else {}))
    small = synth.make(workload, n=700, m=513, **({"d": d} if d else {}))
    scale = 1.0
    if workload == 3:
        scale = 1.0 / sk.mean_sqeuclid(_t(big.x), _t(big.y))
    rng = np.random.default_rng(5)
    with sk.Problem(_t(big.x), _t(big.y), _t(big.a), _t(big.b), scale) as P:
        f, g = _potentials(sk, P, eps, big.n, big.m)
        rows = _t(rng.integers(0, big.n, 4096).astype(np.int64))  # the largest call allowed
        _both(sk, P, eps, f, g, rows, big.m)
        rows = _t(rng.permutation(big.n)[:37].astype(np.int64))  # then a smaller one
        _both(sk, P, eps, f, g, rows, big.m)
    # a second handle with fewer columns right after: the shared array still
    # holds the larger calls' values
    with sk.Problem(_t(small.x), _t(small.y), _t(small.a), _t(small.b), scale) as P:
        f, g = _potentials(sk, P, eps, small.n, small.m)
        rows = _t(np.array([0, small.n - 1, 5, 5, 300], np.int64))
        _both(sk, P, eps, f, g, rows, small.m)


def test_noalloc_refuses_sizes_beyond_its_limits(sk):
    c = synth.make(2, n=5000, m=64)
    with sk.Problem(_t(c.x), _t(c.y), _t(c.a), _t(c.b), 1.0) as P:
        f = torch.zeros(c.n, device=DEV)
        g = torch.zeros(c.m, device=DEV)
        rows = torch.arange(4097, dtype=torch.int64, device=DEV)
        T = torch.zeros((4097, c.m), device=DEV)
        with pytest.raises(sk.SinkhornError) as e:
            P.materialize_rows_noalloc(1e-2, f, g, rows, T)
        assert e.value.code == sk.ERR_INVALID_ARG and "4096" in str(e.value)
        assert float(T.abs().max()) == 0.0  # nothing written
        # a bad row index is refused as by materialize_rows
        rows = torch.tensor([0, 5000], dtype=torch.int64, device=DEV)
        with pytest.raises(sk.SinkhornError) as e:
            P.materialize_rows_noalloc(1e-2, f, g, rows, torch.zeros((2, c.m), device=DEV))
        assert e.value.code == sk.ERR_INVALID_ARG
    wide = synth.make(2, n=8, m=(1 << 21) + 1)
    with sk.Problem(_t(wide.x), _t(wide.y), None, None, 1.0) as P:
        f = torch.zeros(wide.n, device=DEV)
        g = torch.zeros(wide.m, device=DEV)
        rows = torch.arange(2, dtype=torch.int64, device=DEV)
        with pytest.raises(sk.SinkhornError) as e:
            P.materialize_rows_noalloc(1e-2, f, g, rows, torch.zeros((2, wide.m), device=DEV))
        assert e.value.code == sk.ERR_INVALID_ARG and "columns" in str(e.value)
