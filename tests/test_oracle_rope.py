"""Pins for the oracle's 3D RoPE (notes page section 5.5, RoFormer rotation).

Each test checks something the pages or the mathematics fix independently of
the oracle's own code path:

* closed-form angles: theta^(-2j/d) is exactly 1/100 (theta=10000) or 1/16
  (theta=256) when 2j/d = 1/2, and 1 for j = 0;
* the (16, 56, 56) channel blocks: a coordinate along one axis moves only
  that axis's channels;
* identity at the origin, composition R(a)R(b) = R(a+b);
* norm preservation per pair and per head vector;
* the relative-position property: <R(p)q, R(p')k> depends on p - p' only;
* the complex-number form of RoFormer (pair (x0, x1) as x0 + i x1 times
  e^{i phi}), evaluated with Python's cmath row by row;
* text rows are left untouched.
"""
import cmath
import math

import numpy as np
import pytest

from oracle import apply_rope3d, token_grid, video_coordinates

# a small 3 x 4 x 5 token grid: F=9 -> T'=3, H=64 -> 4, W=80 -> 5
GRID = token_grid(9, 64, 80)
TEXT = 7
L = GRID.n_video + TEXT


def tok(t, h, w):
    """Sequence position of patch (t, h, w): time-major, then rows, then columns."""
    return t * (4 * 5) + h * 5 + w


def test_coordinate_table():
    assert GRID.n_video == 60
    coords = video_coordinates(GRID)
    # hand-listed flatten order of the 3x4x5 grid
    expected = {0: (0, 0, 0), 1: (0, 0, 1), 4: (0, 0, 4), 5: (0, 1, 0), 19: (0, 3, 4),
                20: (1, 0, 0), 27: (1, 1, 2), 59: (2, 3, 4)}
    for n, c in expected.items():
        assert tuple(coords[n]) == c
        assert tok(*c) == n


def rot_one(x_row, n, theta):
    x = np.zeros((1, 1, 24, 128))
    x[0, 0] = x_row
    return apply_rope3d(x, np.array([n]), GRID, theta)[0, 0]


@pytest.mark.parametrize("theta,freq", [(10000.0, 0.01), (256.0, 1.0 / 16.0)])
@pytest.mark.parametrize("axis_off,d,coord", [(0, 16, (2, 0, 0)), (16, 56, (0, 3, 0)), (72, 56, (0, 0, 4))])
def test_closed_form_angles(theta, freq, axis_off, d, coord):
    pos = max(coord)
    n = tok(*coord)
    for j, f in ((0, 1.0), (d // 4, freq)):
        # 2j/d = 1/2 for j = d/4
        x = np.zeros((24, 128))
        x[:, axis_off + 2 * j] = 1.0
        y = rot_one(x, n, theta)
        assert np.allclose(y[:, axis_off + 2 * j], math.cos(pos * f), atol=1e-14)
        assert np.allclose(y[:, axis_off + 2 * j + 1], math.sin(pos * f), atol=1e-14)
        # the second basis vector of the pair goes to (-sin, cos)
        x = np.zeros((24, 128))
        x[:, axis_off + 2 * j + 1] = 1.0
        y = rot_one(x, n, theta)
        assert np.allclose(y[:, axis_off + 2 * j], -math.sin(pos * f), atol=1e-14)
        assert np.allclose(y[:, axis_off + 2 * j + 1], math.cos(pos * f), atol=1e-14)


@pytest.mark.parametrize("coord,block", [((2, 0, 0), (0, 16)), ((0, 3, 0), (16, 72)), ((0, 0, 4), (72, 128))])
def test_axis_blocks(coord, block):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((24, 128))
    y = rot_one(x, tok(*coord), 10000.0)
    lo, hi = block
    changed = np.nonzero(np.any(np.abs(y - x) > 0, axis=0))[0]
    assert changed.min() >= lo and changed.max() < hi
    # every pair in the block actually moves (all frequencies are non-zero)
    moved = np.abs(y[:, lo:hi] - x[:, lo:hi]).max(axis=0)
    assert np.all(moved[0::2] + moved[1::2] > 0)


def test_origin_is_identity():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((24, 128))
    assert np.array_equal(rot_one(x, 0, 10000.0), x)


def test_composition():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 1, 24, 128))
    a, b = (1, 1, 1), (1, 2, 3)
    ab = tuple(i + j for i, j in zip(a, b))
    ya = apply_rope3d(x, np.array([tok(*a)]), GRID, 10000.0)
    yab = apply_rope3d(ya, np.array([tok(*b)]), GRID, 10000.0)
    direct = apply_rope3d(x, np.array([tok(*ab)]), GRID, 10000.0)
    assert np.allclose(yab, direct, atol=1e-12)


def test_norm_preserved():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, L, 24, 128))
    y = apply_rope3d(x, np.arange(L), GRID, 10000.0)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    pair_x = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    pair_y = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(pair_x, pair_y, rtol=1e-12)


def test_relative_position():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 24, 128))
    k = rng.standard_normal((1, 1, 24, 128))

    def score(pq, pk):
        rq = apply_rope3d(q, np.array([tok(*pq)]), GRID, 10000.0)[0, 0]
        rk = apply_rope3d(k, np.array([tok(*pk)]), GRID, 10000.0)[0, 0]
        return np.einsum("hd,hd->h", rq, rk)

    base = score((0, 1, 0), (1, 0, 2))
    for shift in ((1, 0, 0), (0, 2, 1), (1, 1, 2)):
        pq = (0 + shift[0], 1 + shift[1], 0 + shift[2])
        pk = (1 + shift[0], 0 + shift[1], 2 + shift[2])
        assert np.allclose(score(pq, pk), base, atol=1e-11)
    # and it does depend on the difference
    assert not np.allclose(score((0, 1, 0), (1, 0, 3)), base, atol=1e-6)


def test_complex_form_matches():
    """RoFormer's complex form: pair (x0, x1) as x0 + i x1, multiplied by e^{i phi}."""
    rng = np.random.default_rng(6)
    theta = 10000.0
    x = rng.standard_normal((1, L, 24, 128))
    y = apply_rope3d(x, np.arange(L), GRID, theta)
    blocks = ((0, 16, 0), (16, 56, 1), (72, 56, 2))
    for n in (1, 7, 23, 44, 59):
        t, h, w = n // 20, (n // 5) % 4, n % 5
        pos = (t, h, w)
        for head in (0, 11, 23):
            for off, d, ax in blocks:
                for j in range(d // 2):
                    z = complex(x[0, n, head, off + 2 * j], x[0, n, head, off + 2 * j + 1])
                    zr = z * cmath.exp(1j * pos[ax] * theta ** (-(2.0 * j) / d))
                    assert abs(zr.real - y[0, n, head, off + 2 * j]) < 1e-12
                    assert abs(zr.imag - y[0, n, head, off + 2 * j + 1]) < 1e-12


def test_text_rows_untouched():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, L, 24, 128))
    y = apply_rope3d(x, np.arange(L), GRID, 10000.0)
    assert np.array_equal(y[:, GRID.n_video:], x[:, GRID.n_video:])
    assert not np.allclose(y[:, 1:GRID.n_video], x[:, 1:GRID.n_video])


def test_row_subset_matches_full():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((1, L, 24, 128))
    full = apply_rope3d(x, np.arange(L), GRID, 256.0)
    rows = np.array([0, 3, 21, 59, 60, L - 1])
    sub = apply_rope3d(x[:, rows], rows, GRID, 256.0)
    assert np.array_equal(sub, full[:, rows])
