"""Pins for the Morton oracle: hand-computed codes, a per-bit brute force with
Python integers, and the properties of a stable sort."""
import numpy as np

import oracle
from oracle.morton import BITS, bounding_box


def _brute_code(q):
    d = len(q)
    code = 0
    for b in range(BITS):
        for k in range(d):
            if (int(q[k]) >> b) & 1:
                code += 1 << (d * b + k)
    return code


def test_hand_computed_codes():
    q = np.array([[1, 0, 0], [0, 1, 0], [0, 0, 1], [1, 1, 1], [2, 0, 0], [3, 0, 0], [0, 0, 2]])
    assert oracle.interleave(q).tolist() == [1, 2, 4, 7, 8, 9, 32]
    top = (1 << BITS) - 1
    assert int(oracle.interleave(np.array([[top, top, top]]))[0]) == (1 << 63) - 1
    assert oracle.interleave(np.array([[5, 3]])).tolist() == [0b011011]


def test_interleave_matches_per_bit_brute_force(rng):
    for d in (1, 2, 3):
        q = rng.integers(0, 1 << BITS, size=(200, d))
        codes = oracle.interleave(q)
        assert [int(c) for c in codes] == [_brute_code(r) for r in q]


def test_quantize_corners_and_degenerate_axis():
    x = np.array([[0.0, 2.0, 5.0], [1.0, 2.0, 5.0]], np.float32)
    y = np.array([[0.5, 2.0, 5.0]], np.float32)
    lo, hi = bounding_box(x, y)
    q = oracle.quantize(x, lo, hi)
    assert q[0].tolist() == [0, 0, 0]
    assert q[1].tolist() == [(1 << BITS) - 1, 0, 0]
    assert oracle.quantize(y, lo, hi)[0, 0] == 1 << (BITS - 1)


def test_order_is_a_stable_sort_of_codes(rng):
    x = rng.uniform(0, 1, size=(300, 3)).astype(np.float32)
    x[50] = x[10]  # duplicates must keep their original order
    x[200] = x[10]
    y = rng.normal(0.5, 0.2, size=(250, 3)).astype(np.float32)
    cx, px, cy, py = oracle.morton_order(x, y)
    for codes, perm, k in ((cx, px, 300), (cy, py, 250)):
        assert sorted(perm.tolist()) == list(range(k))
        assert np.all(codes[1:] >= codes[:-1])
    pos = {int(p): i for i, p in enumerate(px)}
    assert pos[10] < pos[50] < pos[200]
    # codes against the brute force on the shared bounding box
    lo, hi = bounding_box(x, y)
    q = oracle.quantize(x, lo, hi)
    assert [int(c) for c in cx] == [_brute_code(q[p]) for p in px]


def test_grid_points_follow_z_order():
    # the 8 corners of a 2x2x2 grid are visited in z-order: axis 0 fastest
    pts = np.array([[i, j, k] for k in (0, 1) for j in (0, 1) for i in (0, 1)], np.float32)
    rev = pts[::-1].copy()
    _, perm, _, _ = oracle.morton_order(rev, pts)
    assert rev[perm].tolist() == pts.tolist()
