"""Handles on separate host threads, each on a stream of its own, solve at the
same time and return the same bits as the same solves run one after another.
What the handles share inside the library is the pair kernels' occupancy
figures (queried once per kernel) and the device-memory accounting; the check
runs in a child process so that those first queries happen concurrently."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, threading
sys.path.insert(0, sys.argv[1])
import numpy as np
import torch
import log_domain_sinkhorn_amd as sk
import synth

dev = "cuda:0"
t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
c2 = synth.make(2, n=3000, m=2500)           # d = 3: VALU pair kernel
c3 = synth.make(3, n=1500, m=1700, d=50)      # d = 50: MFMA pair kernel
start = sk.device_memory()[0]
s3 = 1.0 / sk.mean_sqeuclid(t(c3.x), t(c3.y))
inputs = [(t(c.x), t(c.y), t(c.a), t(c.b), s) for c, s in ((c2, 1.0), (c3, s3))]
scheds = [sk.Schedule(eps_start=1.0, eps_target=1e-2, eps_factor=0.5, iters_per_stage=5, tol=1e-3, max_iters=1000),
          sk.Schedule(0.05, 0.05, tol=1e-3, max_iters=1000)]
torch.cuda.synchronize()

def run(k, out):
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        x, y, a, b, scale = inputs[k]
        with sk.Problem(x, y, a, b, scale) as P:
            f, g, rep = P.solve(scheds[k])
        s.synchronize()
        out[k] = (f.cpu().numpy(), g.cpu().numpy(), rep["iters"])

# two threads per problem, all four at once
res = [{} for _ in range(4)]
ths = [threading.Thread(target=run, args=(k, res[i])) for i, k in enumerate((0, 1, 0, 1))]
for th in ths:
    th.start()
for th in ths:
    th.join()
seq = {}
for k in (0, 1):
    run(k, seq)
for i, k in enumerate((0, 1, 0, 1)):
    f, g, it = res[i][k]
    assert it == seq[k][2], (k, it, seq[k][2])
    assert np.array_equal(f, seq[k][0]) and np.array_equal(g, seq[k][1]), k
    assert np.isfinite(f).all() and np.isfinite(g).all()
assert sk.device_memory()[0] == start  # every handle gave its memory back
print("threads ok", seq[0][2], seq[1][2])
"""


@pytest.mark.gpu
def test_concurrent_handles_on_host_threads_match_sequential_bits():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("concurrent handles: child process", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "threads ok" in r.stdout
