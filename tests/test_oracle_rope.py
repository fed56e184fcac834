"""Pins for RoPE at explicit position ids.

Pinned by properties the rotation must have, not by retyping it: the pairing
and direction of the rotation on unit vectors, composition of rotations,
norm preservation, dependence of q.k on relative position only, and a
d = 2 special case whose angle is the position itself.
"""

import math

import numpy as np

from oracle import rope


def _unit(d, i):
    e = np.zeros(d)
    e[i] = 1.0
    return e


def test_frequencies():
    th = rope.frequencies(8, 10000.0)
    assert th[0] == 1.0
    assert np.allclose(th, [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    assert np.all(np.diff(rope.frequencies(128)) < 0)


def test_position_zero_is_identity():
    c, s = rope.table(4, 16)
    x = np.random.default_rng(0).standard_normal((3, 16))
    assert np.array_equal(rope.rotate(x, np.zeros(3, int), c, s), x)


def test_d2_angle_is_the_position():
    c, s = rope.table(8, 2)
    out = rope.rotate(np.array([[1.0, 0.0]]), np.array([5]), c, s)[0]
    assert abs(out[0] - math.cos(5.0)) < 1e-7 and abs(out[1] - math.sin(5.0)) < 1e-7


def test_pairs_are_interleaved_and_rotate_counterclockwise():
    d, pos = 8, 3
    c, s = rope.table(8, d)
    th = rope.frequencies(d)
    for i in range(d // 2):
        out = rope.rotate(_unit(d, 2 * i)[None], np.array([pos]), c, s)[0]
        want = np.zeros(d)
        want[2 * i] = math.cos(pos * th[i])
        want[2 * i + 1] = math.sin(pos * th[i])          # e_{2i} turns towards e_{2i+1}
        assert np.allclose(out, want, atol=1e-7)
        out = rope.rotate(_unit(d, 2 * i + 1)[None], np.array([pos]), c, s)[0]
        want = np.zeros(d)
        want[2 * i] = -math.sin(pos * th[i])
        want[2 * i + 1] = math.cos(pos * th[i])
        assert np.allclose(out, want, atol=1e-7)


def test_rotation_preserves_norm():
    c, s = rope.table(6000, 128)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((500, 128))
    pos = rng.integers(0, 6000, 500)
    r = rope.rotate(x, pos, c, s)
    # c, s are fp32-rounded, so c^2 + s^2 = 1 only to ~2**-23
    assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(x, axis=1), rtol=2e-7)


def test_rotations_compose():
    c, s = rope.table(4000, 64)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 64))
    p1 = rng.integers(0, 2000, 50)
    p2 = rng.integers(0, 2000, 50)
    twice = rope.rotate(rope.rotate(x, p1, c, s), p2, c, s)
    once = rope.rotate(x, p1 + p2, c, s)
    assert np.allclose(twice, once, atol=2e-6)


def test_scores_depend_on_relative_position_only():
    c, s = rope.table(9000, 128)
    rng = np.random.default_rng(3)
    q = rng.standard_normal((40, 128))
    k = rng.standard_normal((40, 128))
    pq = rng.integers(0, 4000, 40)
    pk = rng.integers(0, 4000, 40)
    a = np.einsum("nd,nd->n", rope.rotate(q, pq, c, s), rope.rotate(k, pk, c, s))
    b = np.einsum("nd,nd->n", rope.rotate(q, pq + 4321, c, s), rope.rotate(k, pk + 4321, c, s))
    assert np.allclose(a, b, atol=5e-5)


def test_head_axis_broadcast():
    c, s = rope.table(100, 16)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((7, 3, 16))
    pos = rng.integers(0, 100, 7)
    r = rope.rotate(x, pos, c, s)
    for h in range(3):
        assert np.array_equal(r[:, h], rope.rotate(x[:, h], pos, c, s))
