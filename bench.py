#!/usr/bin/env python3
"""Throughput of the online log-domain Sinkhorn hot path on one MI355X.

Default workload (the one the headline metric is quoted on): n = m = 20000
points in d = 3, each cloud an 8-component Gaussian mixture (sigma 0.05),
Dirichlet(1) weights, squared-Euclidean cost (scale 1), eps annealed from 1.0
by halving (10 full iterations per stage) down to 1e-3, then iterated at 1e-3
until the L1 marginal residual is <= 1e-3.

One step = one full solve from zero potentials: every f- and g-half-step
(online tiled log-sum-exp on the GPU), the fused residual checks and the
schedule. Inputs are resident in HBM before the timed region.

Prints ONE JSON line:
  value      = point pairs evaluated by all half-steps / wall time (pair-evals/s)
  roofline   = the pair-loop kernel against the VALU issue rate of the chip,
               timed by HIP events that each launch's dispatch records at the
               kernel's start and end, in a second run of the same K solves
               (the headline run has no events at all)
  cpu_baseline = the fp64 oracle's half-step on the host cores (bounded sample)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# chip constants (MI355X): 256 CUs, 64 lanes of fp32 VALU issue per CU per clock
CUS = 256
CLOCK_HZ = 2.4e9
VALU_LANES_PER_CU = 64
VALU_PEAK_OPS = CUS * VALU_LANES_PER_CU * CLOCK_HZ  # 3.93e13 lane-ops/s (no packed fp32)
MFMA_F32_PEAK = 157.3e12  # dense fp32 matrix FLOP/s
HBM_PEAK = 8.0e12  # bytes/s

# steps / warmup: defaults per workload (a full solve of 4 or 5 takes minutes).
# roofline: how the second, event-timed region runs (None: the same steps).
WORKLOADS = {
    1: dict(sched=dict(eps_start=0.01, eps_target=0.01, fixed_iters=200), steps=5, warmup=1,
            desc="w1: n=m=1000 d=2, x~U[0,1]^2, y~N(0.5,0.1^2), uniform weights, eps=0.01, 200 iterations"),
    2: dict(sched=dict(eps_start=1.0, eps_target=1e-3, eps_factor=0.5, iters_per_stage=10,
                       tol=1e-3, max_iters=20000), steps=5, warmup=1,
            desc="w2: n=m=20000 d=3, 8-component GMM clouds (sigma 0.05), Dirichlet weights, "
                 "eps 1->1e-3 halving x10/stage, then to L1 residual 1e-3"),
    3: dict(sched=dict(eps_start=0.05, eps_target=0.05, tol=1e-3, max_iters=20000), steps=2, warmup=1,
            scale="mean", materialize=1024,
            desc="w3: n=50000 m=60000 d=50, 20-cluster anisotropic GMM (PCA-embedding-like), uniform weights, "
                 "cost / mean cost, eps=0.05 to L1 residual 1e-3, then every plan row materialized in batches "
                 "of 1024 and min_i max_j T_ij"),
    4: dict(sched=dict(eps_start=1.0, eps_target=1e-4, eps_factor=0.5, iters_per_stage=10,
                       tol=1e-3, max_iters=20000), steps=1, warmup=0,
            roofline=dict(eps_start=1e-4, eps_target=1e-4, fixed_iters=5),
            desc="w4: n=m=1e6 d=3, x~U[0,1]^3, y=jittered 100^3 grid, uniform weights, "
                 "eps 1->1e-4 halving x10/stage, then to L1 residual 1e-3"),
    5: dict(multiscale=dict(B=128, eps=1e-4, tol=1e-2), steps=1, warmup=0, roofline=dict(max_fine=3),
            desc="w5: n=m=2^24 d=3, 64-component GMM in [0,1]^3 (sigma U[0.01,0.05]), y = shifted means, "
                 "uniform weights; Morton order, B=128 blocks, cells <= 2x blocks, coarse annealed centroid "
                 "solve + lift, fine loop on block pairs screened with block potential maxima "
                 "(delta_rel = 1e-3/NB), eps=1e-4, to certified L1 residual 1e-2"),
}


def ops_per_pair(d: int) -> int:
    """Vector-ALU instructions per pair that the difference-form half-step
    needs with a fixed per-row shift: d subs and d fmas for the shifted squared
    distance (the shift folded into the first fma), 1 fma for the exponent and
    1 add into the sum. The exp2 of each pair issues on the transcendental unit
    alongside and is not counted against the VALU issue rate."""
    return 2 * d + 2


KERNEL_SOURCES = ("dense.hip", "pairloop.h", "rowfinal.h", "internal.h", "launch_plan.h")

# HBM traffic of a workload's dominant kernel: the committed rocprofv3 PMC
# summary and the sources that kernel is built from (the figure is used only
# while their digest matches the one recorded with the counters)
PMC_RECORDS = {
    2: ("k_lse_valu_w2_n20000_d3_pmc.md", KERNEL_SOURCES),
    3: ("k_lse_mfma_w3_n50000_m60000_d50_pmc.md", ("mfma.hip", "rowfinal.h", "internal.h")),
}


def kernel_source_digest(sources=KERNEL_SOURCES) -> str:
    """sha256 over the sources a pair kernel is built from."""
    import hashlib

    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "log_domain_sinkhorn_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def pmc_traffic(kernel: str, workload: int = 2):
    """HBM bytes per launch of `kernel` from the workload's committed PMC
    summary, or None when there is none or the kernel source changed since it
    was taken."""
    import re

    if workload not in PMC_RECORDS:
        return None
    name, sources = PMC_RECORDS[workload]
    path = os.path.join(ROOT, "profiles", name)
    try:
        text = open(path).read()
        digest = kernel_source_digest(sources)
    except OSError:
        return None
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)\s+kernel_sources_sha256:\s*([0-9a-f]+)\s+kernel:\s*(\S+)", text)
    if not m or m.group(2) != digest or m.group(3) != kernel:
        return None
    return float(m.group(1))


def cpu_baseline(c, eps, scale=1.0, budget_s=12.0):
    """The fp64 oracle's f-half-step, timed on the host cores: whole half-steps
    repeated until the budget is spent, or a leading row block of one when a
    whole half-step would take longer."""
    import numpy as np

    threads = min(16, os.cpu_count() or 1)
    os.environ["ORACLE_THREADS"] = str(threads)
    import oracle

    g = np.zeros(c.m)
    rows = np.arange(min(c.n, 64))
    t = time.perf_counter()
    oracle.halfstep_f(c.x, c.y, c.b, g, eps, scale, rows=rows)
    dt = max(time.perf_counter() - t, 1e-3)
    k = int(min(c.n, max(64, len(rows) * budget_s / dt)))
    rows = None if k == c.n else np.arange(k)
    reps = 0
    t = time.perf_counter()
    while True:
        oracle.halfstep_f(c.x, c.y, c.b, g, eps, scale, rows=rows)
        reps += 1
        dt = time.perf_counter() - t
        if dt >= budget_s or rows is not None:
            break
    what = f"{reps} whole" if rows is None else f"the first {k} of {c.n} rows of one"
    return {
        "value": reps * k * c.m / dt,
        "unit": "pair-evals/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{what} fp64 f-half-step(s), {c.n} x {c.m} pairs each, explicit cost matrix "
                  f"in row chunks over {threads} threads ({dt:.1f} s)",
    }


def copy_calibration(mib: int, reps: int = 5):
    """A plain device copy of `mib` MiB (reads and writes that many bytes per
    launch) for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default per workload)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default per workload)")
    ap.add_argument("--workload", type=int, default=2, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="no HIP events on the pair-kernel launches (no roofline)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--verify", action="store_true",
                    help="workload 5: verify the screened tiles (exact shares) before each fine update")
    ap.add_argument("--adaptive", action="store_true",
                    help="workload 5: sampled lift checks between batches of coarse updates")
    ap.add_argument("--max-fine", type=int, default=None,
                    help="workload 5: cap on fine updates (profiling runs; the default runs to the certificate)")
    ap.add_argument("--roofline-only", action="store_true",
                    help="run only the kernel-timing region once and print its kernel timing (counter runs)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is not built)", file=sys.stderr)
        sys.exit(2)
    if (args.verify or args.adaptive) and "multiscale" not in WORKLOADS[args.workload]:
        print("bench.py: --verify and --adaptive apply to the multiscale workload (5) only", file=sys.stderr)
        sys.exit(2)

    import torch

    import log_domain_sinkhorn_amd as sk
    import synth

    W = WORKLOADS[args.workload]
    if args.steps is None:
        args.steps = W["steps"]
    if args.warmup is None:
        args.warmup = W["warmup"]
    c = synth.make(args.workload)
    dev = torch.device("cuda:0")
    x, y = torch.from_numpy(c.x).to(dev), torch.from_numpy(c.y).to(dev)
    a, b = torch.from_numpy(c.a).to(dev), torch.from_numpy(c.b).to(dev)
    # the cost scale is resolved once, as a number, before anything is timed
    scale = 1.0 / sk.mean_sqeuclid(x, y) if W.get("scale") == "mean" else 1.0
    multiscale = "multiscale" in W
    if multiscale:
        prm = sk.MultiscaleParams(**W["multiscale"])
        if args.max_fine is not None:
            prm.max_fine = args.max_fine
        prm.verify = bool(args.verify)
        prm.adaptive = bool(args.adaptive)
        eps = prm.eps
        kind = sk.PROF_SPARSE
    else:
        sched = sk.Schedule(**W["sched"])
        eps = float(W["sched"]["eps_target"])
        kind = sk.PROF_DENSE
    P = sk.Problem(x, y, a, b, scale)
    f = torch.zeros(c.n, dtype=torch.float32, device=dev)
    g = torch.zeros(c.m, dtype=torch.float32, device=dev)
    batch = W.get("materialize", 0)
    if batch:
        T = torch.empty((batch, c.m), dtype=torch.float32, device=dev)
        rmax = torch.empty(batch, dtype=torch.float32, device=dev)
        row_ids = torch.arange(c.n, dtype=torch.int64, device=dev)

    def step(timing=False, bounded=False, warm=False):
        if not warm:
            f.zero_()
            g.zero_()
        P.profile_enable(kind if timing else 0)
        if multiscale:
            q = prm
            if bounded and "roofline" in W:
                q = sk.MultiscaleParams(**{**prm.__dict__, **W["roofline"]})
            f_, g_, rep = P.solve_multiscale(q, f, g)
            f.copy_(f_)
            g.copy_(g_)
            rep = dict(rep, pairs_evaluated=rep["pairs_evaluated"], seconds=rep["seconds_total"])
        else:
            sc = sk.Schedule(**W["roofline"]) if bounded and "roofline" in W else sched
            _, _, rep = P.solve(sc, f, g)
        kt = P.profile_read() if timing else None
        P.profile_enable(0)
        mat = None
        if batch:
            # every plan row, batch by batch; min over rows of the row maxima
            P.profile_enable(sk.PROF_MATERIALIZE if timing else 0)
            lo = torch.full((), float("inf"), device=dev)
            for r0 in range(0, c.n, batch):
                k = min(batch, c.n - r0)
                P.materialize_rows(eps, f, g, row_ids[r0:r0 + k], T=T[:k], row_max=rmax[:k])
                lo = torch.minimum(lo, rmax[:k].min())
            mat = (lo, P.profile_read() if timing else None)
            P.profile_enable(0)
        return rep, kt, mat

    if args.roofline_only:
        # only the kernel-timing region, once (for counter runs of the large
        # workloads); from zero potentials
        _, kt, _ = step(timing=True, bounded=True)
        ms, nl, pairs = kt
        print(json.dumps({"roofline_only": True, "workload": args.workload,
                          "region": W.get("roofline", "the whole step"),
                          "pair_kernel": {"launches": nl, "avg_ms": ms / max(nl, 1),
                                          "pair_evals_per_s": pairs / (ms * 1e-3) if ms else None}}),
              flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, nothing else on the stream
    reps = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        reps.append(step())
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0

    # second timed region for the roofline: the same steps (workloads 4 and 5:
    # a bounded run of the same kernels) with a HIP event pair recorded by the
    # dispatch of every pair-kernel (and materializer) launch at the kernel's
    # start and end; the events stay out of the first region. The bounded
    # dense run (workload 4) starts from the potentials the timed solve
    # returned, the state most of its half-steps run in (from zero potentials
    # at the target eps the row shifts are poor and more chunks are redone);
    # the bounded multiscale run starts from zero like the solve.
    kernel_ms, launches, kpairs = 0.0, 0, 0.0
    mat_ms, mat_launches, mat_pairs = 0.0, 0, 0.0
    if not args.no_kernel_timing:
        warm = not multiscale and "roofline" in W
        for _ in range(args.steps):
            _, kt, mat = step(timing=True, bounded=True, warm=warm)
            kernel_ms += kt[0]
            launches += kt[1]
            kpairs += kt[2]
            if mat:
                mat_ms += mat[1][0]
                mat_launches += mat[1][1]
                mat_pairs += mat[1][2]
    timed = launches > 0 and kernel_ms > 0

    solve_pairs = sum(r[0]["pairs_evaluated"] for r in reps)
    mat_entries = (c.n * c.m if batch else 0) * args.steps
    value = (solve_pairs + mat_entries) / elapsed
    last = reps[-1][0]
    out = {
        "metric": "pair-evals/s per Sinkhorn half-step (n*m/t) + wall-time to L1 residual 1e-3",
        "value": value,
        "unit": "pair-evals/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": W["desc"],
            "n": c.n,
            "m": c.m,
            "d": c.d,
            "cost_scale": scale,
            "step": ("one multiscale solve (Morton order, cells, coarse solve, lift, fine loop) to the "
                     "certified stop" if multiscale else "one solve from zero potentials to the stop test")
                    + (", then all plan rows materialized" if batch else ""),
        },
        "wall_time_to_residual_s": sum(r[0]["seconds"] for r in reps) / len(reps),
    }
    if multiscale:
        for k in ("certified", "coarse_iters", "fine_updates", "ncells_x", "ncells_y", "last_tiles",
                  "last_candidates", "R_A_row", "R_A_col", "omega", "seconds_sort", "seconds_coarse",
                  "seconds_lift", "seconds_fine"):
            out[k] = last[k]
        out["verify"] = bool(prm.verify)
        out["adaptive"] = bool(prm.adaptive)
        if prm.adaptive:
            out.update(accepted_by_sample=bool(last["accepted_by_sample"]), checks=last["checks"],
                       last_check=dict(zip(("row", "row_se", "col", "col_se"), last["last_check"]),
                                       samples=last["last_check_samples"]))
    else:
        out.update(halfsteps_per_solve=last["halfsteps"], iters_per_solve=last["iters"],
                   final_row_l1=last["row_l1"], final_col_l1=last["col_l1"])
    if "roofline" in W and timed:
        out["roofline_region"] = ("bounded run of the same kernels: " + json.dumps(W["roofline"]))
    if batch:
        out["min_row_max"] = float(reps[-1][2][0])
    mfma = c.d > 8
    if timed:
        out["pair_kernel"] = {
            "launches": launches,
            "avg_ms": kernel_ms / launches,
            "pairs_per_launch": kpairs / launches,
            "pair_evals_per_s": kpairs / (kernel_ms * 1e-3),
        }
        if mfma:
            kp = (c.d + 1 + 3) // 4 * 4
            flops = 2.0 * c.d  # the cross term x . y, algorithmic
            achieved = kpairs * flops / (kernel_ms * 1e-3)
            out["roofline"] = {
                "bound": "mfma",
                "achieved": achieved / 1e12,
                "peak": MFMA_F32_PEAK / 1e12,
                "unit": "TFLOP/s",
                "frac": achieved / MFMA_F32_PEAK,
                "traffic": pmc_traffic(f"k_lse_mfma<{kp}>", args.workload),
                "flops_per_pair": flops,
                "kernel": f"k_lse_mfma<{kp}>",
            }
        else:
            kname = f"k_lse_sparse<{c.d},true>" if multiscale else f"k_lse_valu<{c.d},true>"
            ops = ops_per_pair(c.d)
            achieved = kpairs * ops / (kernel_ms * 1e-3)
            out["roofline"] = {
                "bound": "alu",
                "achieved": achieved / 1e12,
                "peak": VALU_PEAK_OPS / 1e12,
                "unit": "Tops/s",
                "frac": achieved / VALU_PEAK_OPS,
                "traffic": pmc_traffic(kname, args.workload),
                "ops_per_pair": ops,
                "pair_peak": VALU_PEAK_OPS / ops,
                "kernel": kname,
            }
        if mat_launches:
            wbytes = mat_pairs * 4.0
            out["materializer"] = {
                "launches": mat_launches,
                "avg_ms": mat_ms / mat_launches,
                "entries_per_launch": mat_pairs / mat_launches,
                "write_GBps": wbytes / (mat_ms * 1e-3) / 1e9,
                "hbm_frac": wbytes / (mat_ms * 1e-3) / HBM_PEAK,
            }
    if batch and not args.no_kernel_timing:
        # the consumer of the row materializer: sparsify at min_row on the device
        thr = P.min_row(eps, f, g)
        torch.cuda.synchronize()
        t = time.perf_counter()
        ptr, col, val = P.sparsify(eps, f, g, thr, batch=batch)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t
        out["sparsify"] = {
            "threshold": thr,
            "nnz": int(ptr[-1].item()),
            "seconds": dt,
            "note": "count pass, then the entries (two materializations per batch), min_row threshold",
        }
    if not multiscale and c.d <= 8 and not args.no_kernel_timing:
        # barycentric projection + source gradient at the solved potentials
        # (the f-step's loop with d weighted sums: 2d+2 + d VALU per pair)
        reps_b = 3 if c.n * c.m <= 1e10 else 1
        P.barycentric(eps, g, f_hint=f)  # first call: module load, buffers
        torch.cuda.synchronize()
        P.profile_enable(sk.PROF_BARY)
        for _ in range(reps_b):
            P.barycentric(eps, g, f_hint=f)
        bms, bl, bp = P.profile_read()
        P.profile_enable(0)
        bops = ops_per_pair(c.d) + c.d
        out["barycentric"] = {
            "launches": bl,
            "avg_ms": bms / bl,
            "pair_evals_per_s": bp / (bms * 1e-3),
            "ops_per_pair": bops,
            "valu_frac": bp * bops / (bms * 1e-3) / VALU_PEAK_OPS,
            "kernel": f"k_bary_valu<{c.d},true>",
        }
    P.close()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(c, eps, scale)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
