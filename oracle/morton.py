"""Morton (Z-order) codes and the stable Morton order of two clouds.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FlashSinkhorn 2, §3: Morton sorting makes spatially compact cells and blocks of
consecutive points contiguous. The pages give no bit layout, so the reading
adopted is:
  * one bounding box over x and y together: lo_k = min, hi_k = max per axis;
  * 21 bits per axis: q_k = min(2^21 - 1, floor((p_k - lo_k) * (2^21 / (hi_k - lo_k))))
    in float64, with q_k = 0 on an axis where hi_k == lo_k;
  * interleave with axis 0 at the least significant bit of each group of d
    bits: bit b of axis k goes to bit position d*b + k;
  * sort by (code, original index), i.e. a stable sort of the codes.
"""
from __future__ import annotations

import numpy as np

BITS = 21


def bounding_box(x, y):
    """Per-axis min and max over x and y together (float32 values in float64)."""
    x = np.asarray(x, dtype=np.float32)
    y = np.asarray(y, dtype=np.float32)
    lo = np.minimum(x.min(axis=0), y.min(axis=0)).astype(np.float64)
    hi = np.maximum(x.max(axis=0), y.max(axis=0)).astype(np.float64)
    return lo, hi


def quantize(p, lo, hi) -> np.ndarray:
    """Integer grid coordinates in [0, 2^21 - 1] per axis (int64)."""
    p = np.asarray(p, dtype=np.float32).astype(np.float64)
    q = np.zeros(p.shape, dtype=np.int64)
    for k in range(p.shape[1]):
        span = hi[k] - lo[k]
        if span > 0:
            factor = float(1 << BITS) / span
            v = np.floor((p[:, k] - lo[k]) * factor)
            q[:, k] = np.minimum(v, float((1 << BITS) - 1)).astype(np.int64)
    return q


def interleave(q) -> np.ndarray:
    """Morton code: bit b of axis k goes to position d*b + k (uint64)."""
    q = np.asarray(q, dtype=np.uint64)
    d = q.shape[1]
    code = np.zeros(q.shape[0], dtype=np.uint64)
    for b in range(BITS):
        for k in range(d):
            bit = (q[:, k] >> np.uint64(b)) & np.uint64(1)
            code |= bit << np.uint64(d * b + k)
    return code


def morton_codes(x, y):
    """(codes_x, codes_y) over the shared bounding box of x and y."""
    lo, hi = bounding_box(x, y)
    return interleave(quantize(x, lo, hi)), interleave(quantize(y, lo, hi))


def morton_order(x, y):
    """Sorted codes and permutations for both clouds.

    Returns (codes_x_sorted, perm_x, codes_y_sorted, perm_y) where perm[k] is
    the original index of the k-th point in Morton order; ties keep the
    original index order.
    """
    cx, cy = morton_codes(x, y)
    px = np.lexsort((np.arange(len(cx)), cx)).astype(np.int32)
    py = np.lexsort((np.arange(len(cy)), cy)).astype(np.int32)
    return cx[px], px, cy[py], py
