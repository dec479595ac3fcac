#!/usr/bin/env python3
"""Throughput of the online log-domain Sinkhorn hot path on one MI355X.

Default workload: the largest one, n = m = 2^24 points in d = 3 (64-component
Gaussian mixtures), solved block-sparse and multiscale: Morton order, cells,
annealed coarse solve on the cells, lift, then fine updates on block pairs
screened with block potential maxima, at eps = 1e-4, to the certified L1
marginal residual 1e-2. Other workloads with --workload W (1-4: the dense
online half-step; 3: d = 50 on the fp32 MFMA cross term).

What is timed (inputs resident in HBM, handle initialised):
  * wall_time_to_residual_s: one whole solve from zero potentials to its stop
    test (W = 5: the certificate; W = 1..4: the schedule's residual test);
  * the K timed steps (after W untimed ones), bracketed by synchronizations:
      W = 1, 2, 3: one whole solve per step (3: then every plan row
                   materialized in batches of 1024 and min_row);
      W = 4:       one full iteration (f- then g-half-step) at eps = 1e-4,
                   continuing from the solved potentials;
      W = 5:       one fine update (both tile lists screened, sparse f- and
                   g-half-step, admitted residual), continuing from the
                   certified potentials (warm-started multiscale calls).
  value = n * m * (half-steps in the timed steps) / elapsed: the metric's
  n*m/t per half-step. For W = 5 this counts every half-step as n*m pairs
  (what a dense half-step would evaluate); the pairs the sparse half-steps
  actually visited are reported beside it.

Prints ONE JSON line, with
  roofline     = the dominant kernel against the chip's peak for its
                 instruction mix, from unit counts and clock (256 CUs,
                 2.4 GHz; fp32 vector 157.3 TFLOP/s = 128 FMA lanes per CU per
                 clock, fp64 vector 78.6 = 64; fp32 MFMA 157.3; HBM 8 TB/s),
                 its kernel time taken by HIP events that each launch's own
                 dispatch records at the kernel's start and end;
  issue_ceiling = the same mix measured by the library's probe kernels;
  cpu_baseline = the fp64 oracle's half-step on the host cores (bounded sample).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X: 256 CUs at 2.4 GHz. fp32 vector 157.3 TFLOP/s = 256 * 2.4e9 * 128
# lanes * 2 (FMA); fp64 vector 78.6 TFLOP/s: 64 lanes. Nothing here uses
# packed fp32 instructions: the 128 fp32 lanes per clock are issue slots of
# ordinary VALU instructions, which this part fills beyond 64 per clock when
# the instruction mix allows (the probe kernels reach 5.5e13/s).
CUS = 256
CLOCK_HZ = 2.4e9
FP32_VALU_PEAK = CUS * 128 * CLOCK_HZ  # 7.86e13 fp32 lane-instructions/s
FP64_VALU_PEAK = CUS * 64 * CLOCK_HZ   # 3.93e13 fp64 lane-instructions/s
MFMA_F32_PEAK = 157.3e12  # dense fp32 matrix FLOP/s
HBM_PEAK = 8.0e12  # bytes/s

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
                       tol=1e-3, max_iters=20000), steps=20, warmup=5, continuation=True,
            desc="w4: n=m=1e6 d=3, x~U[0,1]^3, y=jittered 100^3 grid, uniform weights, "
                 "eps 1->1e-4 halving x10/stage, then to L1 residual 1e-3"),
    5: dict(multiscale=dict(B=128, eps=1e-4, tol=1e-2), steps=20, warmup=5,
            desc="w5: n=m=2^24 d=3, 64-component GMM in [0,1]^3 (sigma U[0.01,0.05]), y = shifted means, "
                 "uniform weights; Morton order, B=128 blocks, cells <= 2x blocks, coarse annealed centroid "
                 "solve + lift, fine loop on block pairs screened with block potential maxima "
                 "(delta_rel = 1e-3/NB), eps=1e-4, to certified L1 residual 1e-2"),
}


# Issue slots per pair, in fp32 VALU lane-instruction slots of the chip's fp32
# lane rate: an fp32 VALU instruction takes 1, an fp64 one 2 (the fp64 rate is
# half the fp32 rate) and v_exp_f32 4 (transcendentals issue at a quarter of
# the rate; the probe measures 93% of that alone and shows the exp does not
# overlap the other VALU work). The counts are the arithmetic each form does
# per pair, without loop control, chunk loads or the per-row and per-tile work.
def slots_per_pair(d: int, form: str) -> int:
    """form: 'f32' (the shifted difference form: d sub, d fma, 1 fma for the
    exponent, 1 add, 1 exp2), 'f64' (the same in fp64 up to the exponent: d
    add, d + 1 fma in fp64, 1 conversion, then the exp2 and the fp32 add),
    'split' (the precise dense default: the squared distance in fp32, the
    integer column term minus the integer row shift, 1 fma for the exponent,
    the exp2 and 1 fma of the column weight into the sum), 'local' (the
    tile-local expanded form on the vector ALU: 1 mul and d - 1 fma for the
    dot product, the exp2, 1 fma into the tile sum), 'local_mfma' (the same
    form with the dot products on the matrix cores, as the sparse half-step
    runs it: d K = 1 MFMA steps, 2d flops at the fp32 MFMA rate, which is
    twice the fp32 lane rate, so d slots, plus the exp2 and 1 fma; the
    matrix and vector pipes do not overlap on a SIMD, so the slots add)."""
    if form == "f32":
        return (2 * d + 2) + 4
    if form == "f64":
        return 2 * (2 * d + 1) + 2 + 1 + 4
    if form == "local":
        return (d + 1) + 4
    if form == "split":
        return (2 * d + 3) + 4
    if form == "local_mfma":
        return d + 1 + 4
    raise ValueError(form)


SLOT_TEXT = {
    "f32": "2d+2 fp32 VALU + 1 exp2 (4 slots) per pair",
    "f64": "2d+1 fp64 VALU (2 slots each) + 1 fp64-to-fp32 conversion (2) + 1 fp32 add + 1 exp2 (4) per pair",
    "local": "d+1 fp32 VALU + 1 exp2 (4 slots) per pair",
    "split": "2d+3 fp32 VALU (d sub, 1 mul + d-1 fma, 1 sub, 1 fma, 1 fma into the sum) + 1 exp2 (4 slots) per pair",
    "local_mfma": ("d K = 1 steps of v_mfma_f32_4x4x1_16b_f32 (2d flops at the fp32 MFMA rate = d slots; "
                   "the matrix and vector pipes do not overlap on a SIMD) + 1 exp2 (4 slots) + 1 fp32 fma "
                   "per pair"),
}


KERNEL_SOURCES = ("dense.hip", "pairloop.h", "rowfinal.h", "internal.h", "launch_plan.h")
KERNEL_SOURCES_64 = ("dense64.hip", "pairloop64.h", "pairloop.h", "rowfinal.h", "internal.h",
                     "launch_plan.h")
SPARSE_SOURCES = ("blocks.hip", "pairloop.h", "rowfinal.h", "internal.h", "launch_plan.h")

# HBM traffic of a workload's dominant kernel: the committed rocprofv3 PMC
# summary and the sources that kernel is built from (the figure is used only
# while their digest matches the one recorded with the counters)
PMC_RECORDS = {
    2: ("k_lse_split_w2_n20000_d3_pmc.md", KERNEL_SOURCES_64),
    3: ("k_lse_mfma_w3_n50000_m60000_d50_pmc.md", ("mfma.hip", "rowfinal.h", "internal.h")),
    4: ("k_lse_split_w4_n1000000_d3.md", KERNEL_SOURCES_64),
    5: ("k_lse_sparse_w5_n16777216_eps1e-4_pmc.md", SPARSE_SOURCES),
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


PROBES = ("FMA_F32", "SUB_F32", "FMAC_F32", "EXP_F32", "PAIR_F32", "PAIR_F32_NOEXP", "FMA_F64",
          "ADD_F64", "CVT_F32_F64", "PAIR_F64", "PAIR_TILE_F32", "PAIR_SPLIT_F32", "PAIR_TILE_MFMA")


def issue_rates(kinds=PROBES, iters=200000):
    """Measured issue rates of the probe kernels (lane-instructions/s of the
    counted class, pairs/s for the pair probes), the best of three runs each."""
    import log_domain_sinkhorn_amd as sk

    out = {}
    for name in kinds:
        kind = getattr(sk, "PROBE_" + name)
        it = iters if "PAIR" not in name else iters // 8
        best = max((sk.probe_issue_rate(kind, it) for _ in range(3)), key=lambda r: r[0])
        peak = FP64_VALU_PEAK if name.endswith("F64") and "PAIR" not in name else FP32_VALU_PEAK
        out[name] = {"lane_instr_per_s": best[0], "pairs_per_s": best[1] or None, "kernel_ms": best[2],
                     "frac_of_lane_peak": best[0] / peak}
    return out


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


def note(msg):
    """A progress line on stderr (the run's own steps)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def alu_roofline(kname, pairs, ms, d, form, workload):
    rate = pairs / (ms * 1e-3)
    slots = slots_per_pair(d, form)
    achieved = rate * slots
    return {
        "bound": "alu",
        "achieved": achieved / 1e12,
        "peak": FP32_VALU_PEAK / 1e12,
        "unit": "Tops/s",
        "frac": achieved / FP32_VALU_PEAK,
        "traffic": pmc_traffic(kname, workload),
        "ops_per_pair": slots,
        "ops": f"{slots} fp32 issue slots per pair at d = {d}: " + SLOT_TEXT[form],
        "pair_peak": FP32_VALU_PEAK / slots,
        "kernel": kname,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default per workload)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default per workload)")
    ap.add_argument("--workload", type=int, default=5, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="no HIP events on the pair-kernel launches (no roofline)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--verify", action="store_true",
                    help="workload 5: verify the screened tiles (exact shares) before each fine update")
    ap.add_argument("--adaptive", action="store_true",
                    help="workload 5: sampled lift checks between batches of coarse updates")
    ap.add_argument("--fp32-pairs", action="store_true",
                    help="dense d <= 3 half-steps in the fp32 pair loop (SINKHORN_FLAG_FP32_PAIRS)")
    ap.add_argument("--probe", action="store_true",
                    help="only run the issue-rate probe kernels and print their rates")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the kernel-timing region, from a continuation state reached without "
                         "the full solve (counter runs)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.probe:
        print(json.dumps({"issue_rates": issue_rates(), "fp32_lane_peak": FP32_VALU_PEAK,
                          "fp64_lane_peak": FP64_VALU_PEAK}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is not built)", file=sys.stderr)
        sys.exit(2)
    W = WORKLOADS[args.workload]
    multiscale = "multiscale" in W
    if (args.verify or args.adaptive) and not multiscale:
        print("bench.py: --verify and --adaptive apply to the multiscale workload (5) only", file=sys.stderr)
        sys.exit(2)

    import torch

    import log_domain_sinkhorn_amd as sk
    import synth

    if args.steps is None:
        args.steps = W["steps"]
    if args.warmup is None:
        args.warmup = W["warmup"]
    note(f"workload {args.workload}: generating inputs")
    c = synth.make(args.workload)
    dev = torch.device("cuda:0")
    x, y = torch.from_numpy(c.x).to(dev), torch.from_numpy(c.y).to(dev)
    a, b = torch.from_numpy(c.a).to(dev), torch.from_numpy(c.b).to(dev)
    # the cost scale is resolved once, as a number, before anything is timed
    scale = 1.0 / sk.mean_sqeuclid(x, y) if W.get("scale") == "mean" else 1.0
    flags = sk.FLAG_FP32_PAIRS if args.fp32_pairs else 0
    fp64 = c.d <= 3 and not args.fp32_pairs and not multiscale
    P = sk.Problem(x, y, a, b, scale, flags=flags)
    f = torch.zeros(c.n, dtype=torch.float32, device=dev)
    g = torch.zeros(c.m, dtype=torch.float32, device=dev)
    extra = {}
    continuing = multiscale or bool(W.get("continuation"))
    batch = W.get("materialize", 0)

    if multiscale:
        prm = sk.MultiscaleParams(**W["multiscale"])
        prm.verify = bool(args.verify)
        prm.adaptive = bool(args.adaptive)
        eps = prm.eps
        kind = sk.PROF_SPARSE
        cont = dict(prm.__dict__, warm_start=True, adaptive=False, tol=1e-30)

        def solve_once():
            f.zero_()
            g.zero_()
            return P.solve_multiscale(prm, f, g)

        def run_steps(k):
            # k fine updates from (f, g), continuing in place; the last f-step
            # gives the admitted residual of the returned state
            _, _, rep = P.solve_multiscale(sk.MultiscaleParams(**dict(cont, max_fine=k)), f, g)
            assert rep["fine_updates"] == k, rep["fine_updates"]
            return rep, 2 * k + 1
    else:
        sched = sk.Schedule(**W["sched"])
        eps = float(W["sched"]["eps_target"])
        kind = sk.PROF_DENSE
        if batch:
            T = torch.empty((batch, c.m), dtype=torch.float32, device=dev)
            rmax = torch.empty(batch, dtype=torch.float32, device=dev)
            row_ids = torch.arange(c.n, dtype=torch.int64, device=dev)

        def solve_once():
            f.zero_()
            g.zero_()
            return P.solve(sched, f, g)

        def materialize_all():
            # every plan row, batch by batch, and the min_row threshold
            for r0 in range(0, c.n, batch):
                k = min(batch, c.n - r0)
                P.materialize_rows(eps, f, g, row_ids[r0:r0 + k], T=T[:k], row_max=rmax[:k])
            return P.min_row(eps, f, g)

        if continuing:
            def run_steps(k):
                # k full iterations at eps_target, continuing from (f, g); the
                # count includes the two residual half-steps the solve ends with
                _, _, rep = P.solve(sk.Schedule(eps, eps, fixed_iters=k), f, g)
                return rep, rep["halfsteps"]
        else:
            def run_steps(k):
                hs, rep = 0, None
                for _ in range(k):
                    _, _, rep = solve_once()
                    hs += rep["halfsteps"]
                    if batch:
                        extra["min_row"] = materialize_all()
                return rep, hs

    if args.roofline_only:
        if multiscale:
            solve_once()
        elif continuing:
            P.solve(sk.Schedule(eps, eps, fixed_iters=3), f, g)  # a state at eps_target
        P.profile_enable(kind)
        run_steps(3 if continuing else 1)
        ms, nl, pairs = P.profile_read()
        P.profile_enable(0)
        print(json.dumps({"roofline_only": True, "workload": args.workload,
                          "pair_kernel": {"launches": nl, "avg_ms": ms / max(nl, 1),
                                          "pair_evals_per_s": pairs / (ms * 1e-3) if ms else None}}),
              flush=True)
        return

    # one whole solve from zero potentials: the wall time to the residual
    note("one whole solve to the stop test")
    torch.cuda.synchronize()
    t = time.perf_counter()
    _, _, srep = solve_once()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t
    if batch:
        extra["min_row"] = materialize_all()
    note(f"solve done in {wall:.1f} s; {args.warmup} warm-up and {args.steps} timed steps")

    if args.warmup > 0:
        run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    trep, halfsteps = run_steps(args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    note(f"timed steps done in {elapsed:.1f} s")

    # kernel timing: the same steps again (3 of them for the continuing
    # workloads) with a HIP event pair recorded by the dispatch of every
    # pair-kernel launch at the kernel's start and end
    kt = None
    if not args.no_kernel_timing:
        P.profile_enable(kind)
        run_steps(3 if continuing else 1)
        kt = P.profile_read()
        P.profile_enable(0)

    value = c.n * c.m * halfsteps / elapsed
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
        "dtype": "f64+f32" if fp64 else "f32",
        "data": "synthetic",
        "config": {
            "workload": W["desc"],
            "n": c.n,
            "m": c.m,
            "d": c.d,
            "cost_scale": scale,
            "step": ("one fine update from the certified potentials (both tile lists screened, sparse f- "
                     "and g-half-step, admitted residual)" if multiscale else
                     "one full iteration at eps_target from the solved potentials" if continuing
                     else "one solve from zero potentials to the stop test"
                     + (", then all plan rows materialized and min_row" if batch else "")),
            "pair_arithmetic": ("fp32 pair terms, integer/fp64 split of the column term and shift, fp64 "
                                "potentials (d <= 3)") if fp64 else "fp32",
        },
        "wall_time_to_residual_s": wall,
        "halfsteps_timed": halfsteps,
    }
    if multiscale:
        out["evaluated_pair_evals_per_s"] = trep["pairs_evaluated"] / elapsed
        out["solve"] = {k: srep[k] for k in (
            "certified", "coarse_iters", "fine_updates", "ncells_x", "ncells_y", "last_tiles",
            "last_candidates", "R_A_row", "R_A_col", "omega", "seconds_total", "seconds_sort",
            "seconds_coarse", "seconds_lift", "seconds_fine", "pairs_evaluated", "peak_extra_bytes")}
        out["solve"]["verify"] = bool(prm.verify)
        out["solve"]["adaptive"] = bool(prm.adaptive)
        if prm.adaptive:
            out["solve"].update(accepted_by_sample=bool(srep["accepted_by_sample"]), checks=srep["checks"])
    else:
        out["solve"] = {k: srep[k] for k in ("halfsteps", "iters", "final_iters", "row_l1", "col_l1",
                                              "seconds", "seconds_per_halfstep", "workspace_bytes",
                                              "peak_extra_bytes")}
        out["solve"]["history_tail"] = srep["history"][-5:]
        if "min_row" in extra:
            out["min_row"] = extra["min_row"]
    if kt and kt[1] > 0 and kt[0] > 0:
        ms, nl, pairs = kt
        out["pair_kernel"] = {"launches": nl, "avg_ms": ms / nl, "pairs_per_launch": pairs / nl,
                              "pair_evals_per_s": pairs / (ms * 1e-3)}
        if c.d > 8:
            kp = (c.d + 1 + 3) // 4 * 4
            flops = 2.0 * c.d  # the cross term x . y, algorithmic
            achieved = pairs * flops / (ms * 1e-3)
            out["roofline"] = {"bound": "mfma", "achieved": achieved / 1e12, "peak": MFMA_F32_PEAK / 1e12,
                               "unit": "TFLOP/s", "frac": achieved / MFMA_F32_PEAK,
                               "traffic": pmc_traffic(f"k_lse_mfma<{kp}>", args.workload),
                               "flops_per_pair": flops, "kernel": f"k_lse_mfma<{kp}>"}
        else:
            kname = (f"k_lse_sparse<{c.d},true>" if multiscale else
                     f"k_lse_split<{c.d}>" if fp64 else f"k_lse_valu<{c.d},true>")
            form = "local_mfma" if multiscale else "split" if fp64 else "f32"
            out["roofline"] = alu_roofline(kname, pairs, ms, c.d, form, args.workload)
            # the same instruction mix measured by the probe kernels
            name = "PAIR_TILE_MFMA" if multiscale else "PAIR_SPLIT_F32" if fp64 else "PAIR_F32"
            pr = issue_rates((name,))
            out["issue_ceiling"] = {"probe": name, "pairs_per_s": pr[name]["pairs_per_s"],
                                    "kernel_over_probe": (pairs / (ms * 1e-3)) / pr[name]["pairs_per_s"]}
    P.close()
    if not args.no_cpu_baseline:
        note("cpu baseline (the fp64 oracle on the host)")
        out["cpu_baseline"] = cpu_baseline(c, eps, scale)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
