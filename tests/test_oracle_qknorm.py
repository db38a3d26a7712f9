"""Pins of the fp64 oracle's QK-norm prologue (per-head RMSNorm, then 3D RoPE).

The notes page ("HunyuanVideo 模型结构与数学原理", section 5.4) defines
RMSNorm(x) = gamma * x / sqrt(mean(x^2) + eps) over the d = 128 channels of one
head; section 5.2 keeps separate parameters for the video and text streams.
No page prints a value, so each pin is a property or closed form that a
plausible slip breaks: a sum instead of a mean, a missing square root, eps
outside the root, the wrong reduction axis, gamma on the wrong axis, the text
gamma used for video rows, or RoPE applied before the norm.
"""
import numpy as np
import pytest

from oracle import HEAD_DIM, apply_rope3d, qk_norm_rope3d, rms_norm_heads, token_grid

D = HEAD_DIM


def rng(seed=0):
    return np.random.default_rng(seed)


def test_unit_rms_output():
    # gamma = 1, eps = 0: every head vector comes out with RMS exactly 1
    x = rng(1).standard_normal((3, 7, 24, D)) * 5.0
    y = rms_norm_heads(x, np.ones(D), 0.0)
    rms = np.sqrt(np.mean(y * y, axis=-1))
    assert np.allclose(rms, 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("c", [1e-3, 0.5, 7.25, 300.0])
def test_scale_invariance(c):
    x = rng(2).standard_normal((5, 24, D))
    g = 1.0 + 0.3 * rng(3).standard_normal(D)
    assert np.allclose(rms_norm_heads(c * x, g, 0.0), rms_norm_heads(x, g, 0.0), rtol=1e-13, atol=1e-13)


def test_sign_vector_closed_forms():
    # x = r * u with u a +-1 vector: mean(x^2) = r^2 exactly.
    #  eps = 0       -> y = gamma * u
    #  eps = 3 r^2   -> y = gamma * u / 2       (sqrt(r^2 + 3 r^2) = 2 r)
    #  eps = 8 r^2   -> y = gamma * u / 3
    u = np.where(rng(4).random(D) < 0.5, -1.0, 1.0)
    g = 0.5 + rng(5).random(D)
    for r in (0.125, 1.0, 6.0):
        x = r * u
        assert np.allclose(rms_norm_heads(x, g, 0.0), g * u, rtol=1e-14, atol=0)
        assert np.allclose(rms_norm_heads(x, g, 3 * r * r), g * u / 2, rtol=1e-14, atol=0)
        assert np.allclose(rms_norm_heads(x, g, 8 * r * r), g * u / 3, rtol=1e-14, atol=0)


def test_zero_vector_with_eps_is_zero():
    y = rms_norm_heads(np.zeros((2, 24, D)), np.ones(D), 1e-6)
    assert np.array_equal(y, np.zeros_like(y))


def test_reduction_is_per_head_and_per_row():
    x = rng(6).standard_normal((6, 24, D))
    g = 1.0 + 0.2 * rng(7).standard_normal(D)
    y0 = rms_norm_heads(x, g, 1e-6)
    x2 = x.copy()
    x2[2, 5] *= 40.0          # one head of one row
    x2[4, :, 3] += 9.0        # one channel of every head of another row
    y2 = rms_norm_heads(x2, g, 1e-6)
    keep = np.ones((6, 24), bool)
    keep[2, 5] = False
    keep[4, :] = False
    assert np.array_equal(y0[keep], y2[keep])
    # head (2, 5) was only scaled: its output moves by eps / (2 mean(x^2)) ~ 5e-7
    assert np.allclose(y2[2, 5], y0[2, 5], rtol=2e-6, atol=0)


def test_gamma_acts_per_channel():
    x = rng(8).standard_normal((4, 24, D))
    base = rms_norm_heads(x, np.ones(D), 1e-6)
    for i in (0, 17, 127):
        g = np.zeros(D)
        g[i] = 3.0
        y = rms_norm_heads(x, g, 1e-6)
        assert np.array_equal(y[..., np.arange(D) != i], np.zeros_like(y[..., np.arange(D) != i]))
        assert np.allclose(y[..., i], 3.0 * base[..., i], rtol=1e-14, atol=0)


def _grid_rows():
    g = token_grid(9, 64, 96)      # 3 x 4 x 6 = 72 video tokens
    L = g.n_video + 5
    return g, np.arange(L)


def test_text_rows_use_text_gamma_and_are_not_rotated():
    g, idx = _grid_rows()
    L = idx.size
    u = np.where(rng(9).random((1, L, 24, D)) < 0.5, -1.0, 1.0)
    x = 2.5 * u
    gv = 0.5 + rng(10).random(D)
    gt = 0.5 + rng(11).random(D)
    y = qk_norm_rope3d(x, idx, g, 10000.0, gv, gt, 0.0)
    text = idx >= g.n_video
    assert np.allclose(y[0, text], (gt * u[0, text]), rtol=1e-14, atol=0)
    # gamma_text=None means the video gamma everywhere
    y1 = qk_norm_rope3d(x, idx, g, 10000.0, gv, None, 0.0)
    assert np.allclose(y1[0, text], gv * u[0, text], rtol=1e-14, atol=0)
    assert np.array_equal(y1[0, ~text], y[0, ~text])


def test_norm_comes_before_rope():
    # With x = r u (u = +-1) and eps = 0 the normed head is gamma * u, whose
    # channel pair (2j, 2j+1) has magnitude sqrt(g_2j^2 + g_2j+1^2).  RoPE keeps
    # pair magnitudes, so after norm-then-rotate every video pair has exactly that
    # magnitude; rotate-then-norm would mix u's pair into gamma's unequal weights.
    g, idx = _grid_rows()
    L = idx.size
    u = np.where(rng(12).random((1, L, 24, D)) < 0.5, -1.0, 1.0)
    gv = 0.25 + 2.0 * rng(13).random(D)
    y = qk_norm_rope3d(3.0 * u, idx, g, 10000.0, gv, None, 0.0)
    mag = np.sqrt(y[..., 0::2] ** 2 + y[..., 1::2] ** 2)
    want = np.sqrt(gv[0::2] ** 2 + gv[1::2] ** 2)
    assert np.allclose(mag, np.broadcast_to(want, mag.shape), rtol=1e-13, atol=0)
    # and the video rows are rotated: equal to RoPE of gamma * u, not gamma * u
    video = idx < g.n_video
    rot = apply_rope3d(gv * u, idx, g, 10000.0)
    assert np.allclose(y[0, video], rot[0, video], rtol=1e-13, atol=1e-13)
    assert not np.allclose(y[0, 1:g.n_video], (gv * u)[0, 1:g.n_video])


def test_rotated_output_keeps_unit_rms():
    # gamma = 1, eps = 0: the rotation preserves the head's norm, so the fused
    # output still has RMS 1 on video and text rows alike
    g, idx = _grid_rows()
    x = rng(14).standard_normal((2, idx.size, 24, D)) * 0.3
    y = qk_norm_rope3d(x, idx, g, 256.0, np.ones(D), np.ones(D), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=0, atol=1e-13)
