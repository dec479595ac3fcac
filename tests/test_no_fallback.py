"""The product path computes only in the HIP library: it fails loudly without
the library, never imports the oracle, and keeps working when the oracle and
torch's compute operators are replaced by functions that raise (the pattern
of a monkeypatched forbidden path, moscot #846's tests)."""
import os
import re
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "log_domain_sinkhorn_amd")


def test_binding_fails_loudly_without_the_library(monkeypatch):
    import log_domain_sinkhorn_amd as sk

    monkeypatch.setattr(sk, "_LIB", None)
    monkeypatch.setattr(sk, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libsinkhorn.so"))
    with pytest.raises(ImportError):
        sk.lib()
    with pytest.raises(ImportError):
        sk.device_memory()


def test_package_never_imports_the_oracle():
    code = ("import sys; sys.path.insert(0, %r); import log_domain_sinkhorn_amd as sk; sk.lib(); "
            "print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')))" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "[]", out.stdout


def test_product_sources_do_not_name_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for name in files:
            if name.endswith((".py", ".hip", ".h")):
                text = open(os.path.join(dirpath, name)).read()
                assert not re.search(r"\boracle\b", text), os.path.join(dirpath, name)


@pytest.mark.gpu
def test_gpu_path_runs_with_the_oracle_and_torch_compute_forbidden(monkeypatch):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sys.path.insert(0, ROOT)
    import log_domain_sinkhorn_amd as sk
    import oracle
    import synth

    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    c = synth.make(2, n=3000, m=2500)
    s5 = synth.make(5, n=4096, m=4096)
    x, y, a, b = t(c.x), t(c.y), t(c.a), t(c.b)
    x5, y5, a5, b5 = t(s5.x), t(s5.y), t(s5.a), t(s5.b)
    rows = torch.arange(64, dtype=torch.int64, device=dev)
    T = torch.empty((64, c.m), device=dev)
    torch.cuda.synchronize()

    def forbidden(*_a, **_k):
        raise AssertionError("a forbidden compute path was called")

    for name in dir(oracle):
        if callable(getattr(oracle, name)) and not name.startswith("_"):
            monkeypatch.setattr(oracle, name, forbidden)
    for name in ("logsumexp", "exp", "exp2", "log", "cdist", "matmul", "mm", "bmm", "einsum", "sum",
                 "max", "softmax"):
        monkeypatch.setattr(torch, name, forbidden)
    for name in ("logsumexp", "exp", "exp2", "log", "matmul", "sum", "max", "softmax"):
        monkeypatch.setattr(torch.Tensor, name, forbidden)

    with sk.Problem(x, y, a, b, 1.0) as P:
        g = torch.zeros(c.m, device=dev)
        f, _ = P.halfstep_f(0.01, g)
        g2, _ = P.halfstep_g(0.01, f)
        sched = sk.Schedule(eps_start=1.0, eps_target=1e-2, eps_factor=0.5, iters_per_stage=3, tol=1e-3,
                            max_iters=500)
        f, g, rep = P.solve(sched)
        P.materialize_rows(1e-2, f, g, rows, T=T)
        P.marginal_residual(1e-2, f, g)
    with sk.Problem(x5, y5, a5, b5, 1.0) as P:
        f5, g5, rep5 = P.solve_multiscale(sk.MultiscaleParams(B=128, eps=1e-3, tol=1e-2, max_fine=1))
    monkeypatch.undo()
    assert rep["iters"] > 0 and rep5["fine_updates"] == 1
    assert torch.isfinite(f).all() and torch.isfinite(T).all() and torch.isfinite(f5).all()
