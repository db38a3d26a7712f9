"""Pins for the oracle's joint attention (notes page section 5.2).

* brute force against an independent pure-Python evaluation
  (math.exp / math.fsum) on tiny sequences;
* softmax weights: with one-hot values the output rows are the attention
  weights, which are non-negative, sum to 1 and vanish on padded keys;
* closed forms: uniform keys (or q = 0) give the mean of the valid V rows,
  one valid key gives that key's V row, two keys give a logistic mix with
  logit a*b/sqrt(128) (pins the scale and its sign);
* invariances: permuting (k_j, v_j) pairs, adding a common vector to all
  valid keys;
* masking: NaN / huge values in padded K and V rows change nothing;
* the row-subset and head-subset interfaces agree with the full call;
* the end-to-end hot path applies RoPE before attention.
"""
import math

import numpy as np
import pytest

from oracle import apply_rope3d, hot_path, joint_attention, token_grid

D = 128


def brute(q, k, v, lk, scale):
    """Pure-Python attention for one head: q [L, D], k/v [Lk, D] as lists."""
    out = []
    for qi in q:
        s = [scale * math.fsum(qi[d] * k[j][d] for d in range(D)) for j in range(lk)]
        m = max(s)
        p = [math.exp(x - m) for x in s]
        z = math.fsum(p)
        out.append([math.fsum(p[j] * v[j][d] for j in range(lk)) / z for d in range(D)])
    return out


def test_brute_force_tiny():
    rng = np.random.default_rng(10)
    B, L, H = 2, 13, 24
    n_video, valid = 9, (4, 1)
    q = rng.standard_normal((B, L, H, D))
    k = rng.standard_normal((B, L, H, D))
    v = rng.standard_normal((B, L, H, D))
    out = joint_attention(q, k, v, n_video, valid)
    scale = 1.0 / math.sqrt(128.0)
    for b in range(B):
        lk = n_video + valid[b]
        for h in (0, 5, 23):
            ref = brute(q[b, :, h].tolist(), k[b, :, h].tolist(), v[b, :, h].tolist(), lk, scale)
            assert np.allclose(out[b, :, h], np.array(ref), atol=1e-13, rtol=0)


def test_weights_are_a_distribution():
    rng = np.random.default_rng(11)
    L, H = 40, 24
    n_video, valid = 30, (6,)
    lk = n_video + valid[0]
    q = rng.standard_normal((1, L, H, D)) * 3.0
    k = rng.standard_normal((1, L, H, D))
    v = np.zeros((1, L, H, D))
    for j in range(L):
        v[0, j, :, j] = 1.0        # one-hot values: output = weight row
    w = joint_attention(q, k, v, n_video, valid)
    assert np.all(w >= 0)
    assert np.allclose(w[..., :L].sum(axis=-1), 1.0, atol=1e-13)
    assert np.all(w[..., lk:] == 0)


def test_uniform_keys_give_mean():
    rng = np.random.default_rng(12)
    L, H = 20, 24
    n_video, valid = 15, (3,)
    lk = n_video + valid[0]
    q = rng.standard_normal((1, L, H, D))
    k = np.broadcast_to(rng.standard_normal((1, 1, H, D)), (1, L, H, D)).copy()
    v = rng.standard_normal((1, L, H, D))
    out = joint_attention(q, k, v, n_video, valid)
    mean = v[0, :lk].mean(axis=0)
    assert np.allclose(out[0], mean[None], atol=1e-13)
    # q = 0 also gives the mean, whatever the keys
    k2 = rng.standard_normal((1, L, H, D))
    out2 = joint_attention(np.zeros_like(q), k2, v, n_video, valid)
    assert np.allclose(out2[0], mean[None], atol=1e-13)


def test_single_key():
    rng = np.random.default_rng(13)
    L, H = 5, 24
    q = rng.standard_normal((1, L, H, D)) * 10
    k = rng.standard_normal((1, L, H, D))
    v = rng.standard_normal((1, L, H, D))
    out = joint_attention(q, k, v, 1, (0,))
    assert np.allclose(out[0], v[0, 0][None], atol=1e-15)


@pytest.mark.parametrize("a,b", [(3.0, 2.0), (-4.0, 5.0), (20.0, 20.0)])
def test_two_key_closed_form(a, b):
    L, H = 2, 24
    q = np.zeros((1, L, H, D)); q[..., 0] = a
    k = np.zeros((1, L, H, D)); k[0, 0, :, 0] = b
    rng = np.random.default_rng(14)
    v = rng.standard_normal((1, L, H, D))
    out = joint_attention(q, k, v, 2, (0,))
    p0 = 1.0 / (1.0 + math.exp(-a * b / math.sqrt(128.0)))
    expect = p0 * v[0, 0] + (1.0 - p0) * v[0, 1]
    assert np.allclose(out[0], expect[None], atol=1e-13)


def test_permutation_and_shift_invariance():
    rng = np.random.default_rng(15)
    L, H = 33, 24
    n_video, valid = 25, (5,)
    lk = n_video + valid[0]
    q = rng.standard_normal((1, L, H, D))
    k = rng.standard_normal((1, L, H, D))
    v = rng.standard_normal((1, L, H, D))
    base = joint_attention(q, k, v, n_video, valid)
    perm = np.concatenate([rng.permutation(lk), np.arange(lk, L)])
    assert np.allclose(joint_attention(q, k[:, perm], v[:, perm], n_video, valid), base, atol=1e-13)
    u = rng.standard_normal((1, 1, H, D)) * 4
    k2 = k.copy()
    k2[:, :lk] += u
    assert np.allclose(joint_attention(q, k2, v, n_video, valid), base, atol=1e-12)


def test_masking_ignores_poison():
    rng = np.random.default_rng(16)
    L, H = 30, 24
    n_video, valid = 20, (4,)
    lk = n_video + valid[0]
    q = rng.standard_normal((1, L, H, D))
    k = rng.standard_normal((1, L, H, D))
    v = rng.standard_normal((1, L, H, D))
    base = joint_attention(q, k, v, n_video, valid)
    kp, vp = k.copy(), v.copy()
    kp[:, lk:] = 1e30
    vp[:, lk:] = np.nan
    out = joint_attention(q, kp, vp, n_video, valid)
    assert np.array_equal(out, base)
    # the padded tail really would matter if it were not masked
    alt = joint_attention(q, k, v, n_video, (L - n_video,))
    assert not np.allclose(alt, base)


def test_row_and_head_subsets():
    rng = np.random.default_rng(17)
    B, L, H = 2, 21, 24
    q = rng.standard_normal((B, L, H, D))
    k = rng.standard_normal((B, L, H, D))
    v = rng.standard_normal((B, L, H, D))
    full = joint_attention(q, k, v, 16, (5, 2))
    rows = np.array([0, 7, 15, 16, 20])
    sub = joint_attention(q[:, rows], k, v, 16, (5, 2), heads=[3, 17])
    assert np.allclose(sub, full[:, rows][:, :, [3, 17]], atol=1e-15)


def test_hot_path_applies_rope_first():
    from hvinputs import bf16_bits_to_f64, draw_qkv

    g = token_grid(5, 32, 48)     # 2 x 2 x 3 = 12 video tokens
    L = g.n_video + 6
    bits = draw_qkv(1, L, seed=99)
    grid, out = hot_path(bits["q"], bits["k"], bits["v"], 5, 32, 48, (4,), 10000.0)
    assert grid.n_video == 12
    qf = apply_rope3d(bf16_bits_to_f64(bits["q"]), np.arange(L), g, 10000.0)
    kf = apply_rope3d(bf16_bits_to_f64(bits["k"]), np.arange(L), g, 10000.0)
    ref = joint_attention(qf, kf, bf16_bits_to_f64(bits["v"]), 12, (4,))
    assert np.array_equal(out, ref)
    # without RoPE the answer differs
    plain = joint_attention(bf16_bits_to_f64(bits["q"]), bf16_bits_to_f64(bits["k"]),
                            bf16_bits_to_f64(bits["v"]), 12, (4,))
    assert not np.allclose(plain, ref)


def test_rejects_empty_key_set():
    z = np.zeros((1, 3, 24, D))
    with pytest.raises(ValueError):
        joint_attention(z, z, z, 0, (0,))
