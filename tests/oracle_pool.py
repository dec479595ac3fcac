"""The oracle's block-pair screen over worker processes, for the full-size GPU
checks (2^24 points: 131072 x 131072 block pairs, minutes for one process).

Test infrastructure: it calls ``oracle.screen`` unchanged, on ranges of row
blocks, in spawned processes (they import numpy and the oracle only and hold
no GPU state). Each range comes back as its per-block tile counts and a
SHA-256 of its tile indices, so that a list of hundreds of millions of
entries is compared bit for bit without shipping it between processes.
"""
from __future__ import annotations

import hashlib
import multiprocessing as mp
import os

import numpy as np

import oracle

_STATE = {}


def workers() -> int:
    """Processes for the pool: OMP_NUM_THREADS when set, else the CPUs this
    process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "").strip()
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except (AttributeError, OSError):
        return max(1, os.cpu_count() or 1)


def spans(count: int, width: int):
    return [(s, min(count, s + width)) for s in range(0, count, width)]


def digest(ptr, idx, lo: int, hi: int):
    """(counts, sha256) of rows [lo, hi) of a CSR tile list."""
    ptr = np.asarray(ptr, dtype=np.int64)
    seg = np.ascontiguousarray(np.asarray(idx)[ptr[lo]:ptr[hi]], dtype=np.int32)
    return np.diff(ptr[lo:hi + 1]), hashlib.sha256(seg.tobytes()).hexdigest()


def _init(sx, sy, eps, scale, delta):
    _STATE.update(sx=sx, sy=sy, eps=eps, scale=scale, delta=delta)


def _screen_span(span):
    lo, hi = span
    S = _STATE
    ptr, col = oracle.screen(S["sx"], S["sy"], S["eps"], S["scale"], S["delta"],
                             row_blocks=range(lo, hi))
    counts, h = digest(ptr, col, 0, hi - lo)
    return lo, hi, counts, h


def screen_digests(sx, sy, eps: float, scale: float, delta: float, width: int = 1024, procs=None):
    """[(lo, hi, counts, sha256)] of ``oracle.screen`` over row-block ranges
    of ``width`` blocks, in order."""
    nb = sx[0].shape[0]
    procs = workers() if procs is None else procs
    ctx = mp.get_context("spawn")
    with ctx.Pool(procs, initializer=_init, initargs=(sx, sy, eps, scale, delta)) as pool:
        out = pool.map(_screen_span, spans(nb, width), chunksize=1)
    return sorted(out, key=lambda r: r[0])
