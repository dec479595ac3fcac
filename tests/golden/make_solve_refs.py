"""Write the oracle's annealed-solve results used by the GPU solve-parity tests.

Calls only ``oracle`` and ``synth`` (the seeded generators). Each case stores
the fp64 potentials, the iteration counts and the residuals of the oracle run
in ``tests/golden/solve_<name>.npz``. Regenerate with

    python tests/golden/make_solve_refs.py [name ...]
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

# name: (workload, n, m, schedule kwargs, cost scale rule)
CASES = {
    "w1_full_fixed200": (1, None, None, dict(eps_start=0.01, eps_target=0.01, fixed_iters=200), "one"),
    "w2_n1000_tol": (2, 1000, 1000, dict(eps_start=1.0, eps_target=1e-3, tol=1e-3, max_iters=5000), "one"),
    "w4_n1000_tol": (4, 1000, 1000, dict(eps_start=1.0, eps_target=1e-4, tol=1e-3, max_iters=5000), "one"),
    "w3_n1500_tol": (3, 1500, 1800, dict(eps_start=0.05, eps_target=0.05, tol=1e-3, max_iters=5000), "mean"),
    # the full 20000 x 20000 workload (a few hours of fp64 numpy on a few cores)
    "w2_full_tol": (2, None, None, dict(eps_start=1.0, eps_target=1e-3, tol=1e-3, max_iters=5000), "one"),
    # the full 50000 x 60000, d = 50 workload, a fixed budget of 10 iterations
    # (about 12 minutes of fp64 numpy per iteration on 8 cores)
    "w3_full_fixed10": (3, None, None, dict(eps_start=0.05, eps_target=0.05, fixed_iters=10), "mean"),
}


def run(name):
    w, n, m, kw, rule = CASES[name]
    c = synth.make(w, n=n, m=m)
    scale = 1.0 if rule == "one" else 1.0 / oracle.mean_sqeuclid(c.x, c.y)
    sched = oracle.Schedule(**kw)
    t = time.time()
    r = oracle.solve(c.x, c.y, c.a, c.b, scale, sched)
    out = os.path.join(HERE, f"solve_{name}.npz")
    np.savez_compressed(
        out, f=r.f, g=r.g, iters=r.iters, final_iters=r.final_iters, R_row=r.R_row, R_col=r.R_col,
        converged=r.converged, scale=scale, workload=w, n=c.n, m=c.m,
        eps_start=sched.eps_start, eps_target=sched.eps_target, eps_factor=sched.eps_factor,
        iters_per_stage=sched.iters_per_stage, fixed_iters=sched.fixed_iters, tol=sched.tol,
        max_iters=sched.max_iters,
    )
    print(f"{name}: iters {r.iters} (final {r.final_iters}) R {r.R_row:.3e}/{r.R_col:.3e} "
          f"converged {r.converged} in {time.time() - t:.1f}s -> {out}", flush=True)


def main(names):
    for name in names or list(CASES) + list(FS2_CASES):
        if name in FS2_CASES:
            run_fs2(name)
        else:
            run(name)


# multiscale (block-sparse) solve cases: name -> (workload, n, FS2Params kwargs)
# "fixed": the coarse stage runs all its iterations (no tolerance, no stall)
# and the fine loop runs exactly max_fine updates (tol is unreachable), so
# both sides take the same number of steps.
FS2_CASES = {
    "w5_n16384_fixed": (5, 16384, dict(B=128, eps=1e-3, tol=1e-30, coarse_tol=0.0, coarse_max=40,
                                       stall_window=1 << 30, max_fine=4)),
    "w5_n16384_fixed_verify": (5, 16384, dict(B=128, eps=1e-3, tol=1e-30, coarse_tol=0.0,
                                              coarse_max=40, stall_window=1 << 30, max_fine=4,
                                              verify=True)),
    # adaptive switch with an unreachable tol: both checks (after 20 and 40 centroid updates)
    # fail and expand to the larger sample, then the fine loop runs its fixed budget
    "w5_n16384_adaptive": (5, 16384, dict(B=128, eps=1e-3, tol=1e-30, coarse_tol=0.0, coarse_max=40,
                                          stall_window=1 << 30, max_fine=4, adaptive=True,
                                          check_every=20, check_samples=1024, check_samples_max=8192,
                                          sample_seed=11)),
}


def run_fs2(name):
    from oracle.fs2 import FS2Params

    w, n, kw = FS2_CASES[name]
    c = synth.make(w, n=n, m=n)
    prm = FS2Params(**kw)
    t = time.time()
    r = oracle.fs2_solve(c.x, c.y, c.a, c.b, prm)
    out = os.path.join(HERE, f"fs2_{name}.npz")
    np.savez_compressed(
        out, f=r.f, g=r.g, coarse_iters=r.coarse_iters, fine_updates=r.fine_updates,
        R_A_row=r.R_A_row, R_A_col=r.R_A_col, omega=r.omega, certified=r.certified,
        ncells_x=r.ncells_x, ncells_y=r.ncells_y, tiles=np.asarray(r.tiles_history),
        candidates=np.asarray(r.candidates_history), checks=r.checks,
        check_history=np.asarray(r.check_history, dtype=np.float64).reshape(-1, 5),
        accepted_by_sample=r.accepted_by_sample, workload=w, n=n,
        **{k: v for k, v in prm.__dict__.items()},
    )
    print(f"{name}: coarse {r.coarse_iters} fine {r.fine_updates} certified {r.certified} "
          f"R_A {r.R_A_row:.3e}/{r.R_A_col:.3e} cells {r.ncells_x}/{r.ncells_y} in {time.time() - t:.1f}s -> {out}",
          flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
