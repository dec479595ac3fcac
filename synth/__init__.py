"""Seeded synthetic point clouds for the five benchmark workloads.

This module only draws random inputs (coordinates and weights). It holds none
of the transport arithmetic: no costs, potentials, scalings or sorting. Both
the fp64 oracle and the GPU library read the arrays it returns, so they see
identical bytes.

Conventions (all workloads):
  * ``numpy.random.default_rng(seed)``; draw order is x, then y, then weights.
  * Everything is drawn in float64 and cast to float32 at the end.
  * ``a`` and ``b`` are float32 vectors (uniform weights are 1/n as float32).

Workloads (sizes are the defaults; tests may shrink n and m):
  1. n=m=1000, d=2: x ~ U[0,1]^2, y ~ N((0.5,0.5), 0.1^2 I), uniform weights.
  2. n=m=20000, d=3: each cloud is an 8-component isotropic Gaussian mixture,
     means ~ U[0,1]^3, sigma 0.05, mixing weights ~ Dirichlet(1); weights
     a, b ~ Dirichlet(1) over the points.
  3. n=50000, m=60000, d=50: 20-cluster anisotropic Gaussian mixture, means
     ~ N(0, 2^2 I), per-cluster diagonal std ~ U[0.2, 2], equal mixing; y uses
     the x cluster means shifted by N(0, 0.5^2 I) with the same stds and
     independently drawn labels; uniform weights.
  4. n=m=10^6, d=3: x ~ U[0,1]^3; y = centres of a regular 100^3 grid jittered
     by U[-0.005, 0.005]^3; uniform weights.
  5. n=m=2^24, d=3: x from a 64-component Gaussian mixture, means ~ U[0,1]^3,
     sigma_c ~ U[0.01, 0.05], equal mixing; y uses the means shifted by
     N(0, 0.02^2 I) with the same sigmas and independent labels; uniform
     weights 2^-24.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["Clouds", "make", "DEFAULT_SIZES"]

DEFAULT_SIZES = {
    1: (1000, 1000),
    2: (20000, 20000),
    3: (50000, 60000),
    4: (1_000_000, 1_000_000),
    5: (1 << 24, 1 << 24),
}


@dataclass
class Clouds:
    """Source points x [n,d], target points y [m,d], weights a [n], b [m] (float32)."""

    x: np.ndarray
    y: np.ndarray
    a: np.ndarray
    b: np.ndarray
    workload: int
    seed: int

    @property
    def n(self) -> int:
        return self.x.shape[0]

    @property
    def m(self) -> int:
        return self.y.shape[0]

    @property
    def d(self) -> int:
        return self.x.shape[1]


def _uniform_weights(k: int) -> np.ndarray:
    return np.full(k, 1.0 / k, dtype=np.float64)


def _dirichlet_weights(rng: np.random.Generator, k: int) -> np.ndarray:
    w = rng.dirichlet(np.ones(k))
    return w / w.sum()


def _mixture(rng, k, means, stds, probs):
    """Draw k points from a Gaussian mixture with per-component diagonal stds."""
    labels = rng.choice(len(means), size=k, p=probs)
    noise = rng.standard_normal((k, means.shape[1]))
    return means[labels] + noise * stds[labels]


def _w1(rng, n, m):
    x = rng.uniform(0.0, 1.0, size=(n, 2))
    y = rng.normal(0.5, 0.1, size=(m, 2))
    return x, y, _uniform_weights(n), _uniform_weights(m)


def _w2(rng, n, m):
    pts = []
    for k in (n, m):
        means = rng.uniform(0.0, 1.0, size=(8, 3))
        probs = rng.dirichlet(np.ones(8))
        stds = np.full((8, 3), 0.05)
        pts.append(_mixture(rng, k, means, stds, probs))
    a = _dirichlet_weights(rng, n)
    b = _dirichlet_weights(rng, m)
    return pts[0], pts[1], a, b


def _w3(rng, n, m, d=50):
    means = rng.normal(0.0, 2.0, size=(20, d))
    stds = rng.uniform(0.2, 2.0, size=(20, d))
    probs = np.full(20, 1.0 / 20)
    x = _mixture(rng, n, means, stds, probs)
    shifted = means + rng.normal(0.0, 0.5, size=means.shape)
    y = _mixture(rng, m, shifted, stds, probs)
    return x, y, _uniform_weights(n), _uniform_weights(m)


def _w4(rng, n, m):
    side = int(round(m ** (1.0 / 3.0)))
    if side ** 3 != m:
        raise ValueError(f"workload 4 needs m to be a perfect cube, got {m}")
    x = rng.uniform(0.0, 1.0, size=(n, 3))
    idx = np.arange(m)
    i, j, k = idx // (side * side), (idx // side) % side, idx % side
    centres = (np.stack([i, j, k], axis=1) + 0.5) / side
    half = 0.5 / side
    y = centres + rng.uniform(-half, half, size=(m, 3))
    return x, y, _uniform_weights(n), _uniform_weights(m)


def _w5(rng, n, m):
    means = rng.uniform(0.0, 1.0, size=(64, 3))
    sig = rng.uniform(0.01, 0.05, size=64)
    stds = np.repeat(sig[:, None], 3, axis=1)
    probs = np.full(64, 1.0 / 64)
    x = _mixture(rng, n, means, stds, probs)
    shifted = means + rng.normal(0.0, 0.02, size=means.shape)
    y = _mixture(rng, m, shifted, stds, probs)
    return x, y, _uniform_weights(n), _uniform_weights(m)


_GEN = {1: _w1, 2: _w2, 3: _w3, 4: _w4, 5: _w5}


def make(workload: int, n: int | None = None, m: int | None = None, seed: int | None = None,
         d: int | None = None) -> Clouds:
    """Return the seeded clouds of ``workload`` (1..5), optionally resized.

    The seed defaults to the workload number. Resized clouds keep the same
    recipe (distribution, structure and weight law) at the smaller size;
    ``d`` changes the dimension of workload 3 only (default 50).
    """
    if workload not in _GEN:
        raise ValueError(f"unknown workload {workload}")
    dn, dm = DEFAULT_SIZES[workload]
    n = dn if n is None else int(n)
    m = dm if m is None else int(m)
    seed = workload if seed is None else int(seed)
    rng = np.random.default_rng(seed)
    if d is not None and workload != 3:
        raise ValueError("only workload 3 takes a dimension")
    if workload == 3 and d is not None:
        x, y, a, b = _w3(rng, n, m, d=int(d))
    else:
        x, y, a, b = _GEN[workload](rng, n, m)
    return Clouds(
        x=np.ascontiguousarray(x, dtype=np.float32),
        y=np.ascontiguousarray(y, dtype=np.float32),
        a=np.ascontiguousarray(a, dtype=np.float32),
        b=np.ascontiguousarray(b, dtype=np.float32),
        workload=workload,
        seed=seed,
    )
