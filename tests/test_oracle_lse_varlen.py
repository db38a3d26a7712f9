"""Pins of the fp64 oracle's log-sum-exp attention, partial merge and packed
(variable-length) attention.

The notes page ("HunyuanVideo 模型结构与数学原理") names the two uses: section
9.2 (Ring Attention keeps each rank's query rows and passes K/V blocks, so
per-block results must be combined exactly) and section 9.1 (the model calls
the variable-length FlashAttention entry, i.e. packed segments).  No page
prints a value; the pins are closed forms, the union identity (which holds
for exact attention whatever the merge formula looks like), brute force with
math.fsum, and agreement with the already-pinned joint_attention.
"""
import math

import numpy as np
import pytest

from oracle import attention_lse, joint_attention, merge_partials, token_grid, varlen_attention

D = 128


def rng(seed):
    return np.random.default_rng(seed)


def test_lse_one_key_and_repeated_keys():
    r = rng(1)
    q = r.standard_normal((1, 5, 2, D))
    k = r.standard_normal((1, 1, 2, D))
    v = r.standard_normal((1, 1, 2, D))
    out, lse = attention_lse(q, k, v, [1])
    s = 1.0 / math.sqrt(D)
    for h in range(2):
        assert np.allclose(lse[0, h], s * q[0, :, h] @ k[0, 0, h], rtol=1e-13, atol=1e-13)
        assert np.allclose(out[0, :, h], v[0, 0, h][None, :], rtol=1e-13, atol=1e-13)
    # n copies of one key: log-sum-exp gains log n, the output stays v
    kk = np.repeat(k, 7, axis=1)
    vv = np.repeat(v, 7, axis=1)
    out7, lse7 = attention_lse(q, kk, vv, [7])
    assert np.allclose(lse7, lse + math.log(7), rtol=1e-13, atol=1e-13)
    assert np.allclose(out7, out, rtol=1e-12, atol=1e-13)


def test_lse_brute_force():
    r = rng(2)
    q = r.standard_normal((2, 4, 3, D))
    k = r.standard_normal((2, 9, 3, D))
    v = r.standard_normal((2, 9, 3, D))
    out, lse = attention_lse(q, k, v, [9, 5], scale=0.2)
    for b, n in ((0, 9), (1, 5)):
        for h in range(3):
            for i in range(4):
                logits = [0.2 * math.fsum(q[b, i, h] * k[b, j, h]) for j in range(n)]
                z = math.fsum(math.exp(x) for x in logits)
                assert abs(lse[b, h, i] - math.log(z)) < 1e-12
                for c in (0, 64, 127):
                    ref = math.fsum(math.exp(x) * v[b, j, h, c] for j, x in enumerate(logits)) / z
                    assert abs(out[b, i, h, c] - ref) < 1e-12


def test_lse_out_matches_joint_attention():
    r = rng(3)
    L, N = 70, 60
    q, k, v = (r.standard_normal((2, L, 24, D)) for _ in range(3))
    out, _ = attention_lse(q, k, v, [N + 4, N + 10])
    ref = joint_attention(q, k, v, N, [4, 10])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("cuts", [[40], [1, 2], [10, 20, 30, 61], [64]])
def test_merge_of_key_blocks_equals_attention_over_all(cuts):
    r = rng(4)
    Lk = 65
    q = r.standard_normal((1, 6, 24, D)) * 3.0      # peaky
    k = r.standard_normal((1, Lk, 24, D))
    v = r.standard_normal((1, Lk, 24, D))
    full, lse_full = attention_lse(q, k, v, [Lk])
    bounds = [0] + cuts + [Lk]
    parts = [attention_lse(q, k[:, a:b], v[:, a:b], [b - a]) for a, b in zip(bounds, bounds[1:])]
    out, lse = merge_partials([p[0] for p in parts], [p[1] for p in parts])
    assert np.allclose(out, full, rtol=1e-11, atol=1e-12)
    assert np.allclose(lse, lse_full, rtol=1e-13, atol=1e-12)
    # order of the parts does not matter; one part is the identity
    out_r, lse_r = merge_partials([p[0] for p in parts[::-1]], [p[1] for p in parts[::-1]])
    assert np.allclose(out_r, out, rtol=1e-12, atol=1e-13) and np.allclose(lse_r, lse)
    o1, l1 = merge_partials([full], [lse_full])
    assert np.allclose(o1, full, rtol=1e-14, atol=0) and np.allclose(l1, lse_full, rtol=1e-14, atol=0)


def test_merge_equal_weights_averages():
    r = rng(5)
    a, b = r.standard_normal((2, 1, 3, 24, D))
    lse = np.full((1, 24, 3), 1.25)
    out, l = merge_partials([a, b], [lse, lse])
    assert np.allclose(out, (a + b) / 2, rtol=1e-14, atol=1e-15)
    assert np.allclose(l, 1.25 + math.log(2), rtol=1e-14, atol=0)


def test_varlen_one_segment_is_plain_attention():
    r = rng(6)
    T = 50
    q, k, v = (r.standard_normal((T, 24, D)) for _ in range(3))
    out, lse = varlen_attention(q, k, v, [0, T], [0, T])
    ref, lref = attention_lse(q[None], k[None], v[None], [T])
    assert np.allclose(out, ref[0], rtol=1e-13, atol=1e-14)
    assert np.allclose(lse, lref[0], rtol=1e-13, atol=1e-14)


def test_varlen_clips_equal_separate_joint_calls_and_are_isolated():
    # two clips [video | valid text] of different grids packed back to back
    r = rng(7)
    g1, g2 = token_grid(1, 32, 48), token_grid(5, 32, 32)   # 2x3 = 6 and 2x2x2 = 8 tokens
    clips = [(g1.n_video, 5), (g2.n_video, 9)]
    lens = [n + t for n, t in clips]
    T = sum(lens)
    q, k, v = (r.standard_normal((T, 24, D)) for _ in range(3))
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, lse = varlen_attention(q, k, v, cu, cu)
    for s, (n, t) in enumerate(clips):
        a, b = cu[s], cu[s + 1]
        ref = joint_attention(q[None, a:b], k[None, a:b], v[None, a:b], n, [t])
        assert np.allclose(out[a:b], ref[0], rtol=1e-12, atol=1e-13)
    # changing the second clip's keys and values leaves the first clip unchanged
    k2, v2 = k.copy(), v.copy()
    k2[cu[1]:] += 5.0
    v2[cu[1]:] *= -3.0
    out2, _ = varlen_attention(q, k2, v2, cu, cu)
    assert np.array_equal(out2[:cu[1]], out[:cu[1]])
    assert not np.allclose(out2[cu[1]:], out[cu[1]:])


def test_varlen_padded_batch_reading():
    # A padded batch [B, L] flattened with segments [valid | padded tail] per
    # entry: valid rows equal joint attention over the valid keys; each padded
    # tail attends to itself only; empty tails are empty segments.
    r = rng(8)
    B, N, cap = 2, 12, 6
    L = N + cap
    valid = [2, 6]
    q, k, v = (r.standard_normal((B, L, 24, D)) for _ in range(3))
    cu = [0]
    for b in range(B):
        cu += [b * L + N + valid[b], (b + 1) * L]
    out, lse = varlen_attention(q.reshape(B * L, 24, D), k.reshape(B * L, 24, D),
                                v.reshape(B * L, 24, D), cu, cu)
    out = out.reshape(B, L, 24, D)
    ref = joint_attention(q, k, v, N, valid)
    for b in range(B):
        n = N + valid[b]
        assert np.allclose(out[b, :n], ref[b, :n], rtol=1e-12, atol=1e-13)
        if n < L:
            tail, _ = attention_lse(q[b:b + 1, n:], k[b:b + 1, n:], v[b:b + 1, n:], [L - n])
            assert np.allclose(out[b, n:], tail[0], rtol=1e-12, atol=1e-13)


def test_varlen_rows_outside_segments_stay_zero():
    r = rng(9)
    T = 20
    q, k, v = (r.standard_normal((T, 24, D)) for _ in range(3))
    out, lse = varlen_attention(q, k, v, [0, 7, 7, 15], [0, 7, 9, 15])
    assert not out[15:].any() and not lse[:, 15:].any()
    # the empty second query segment writes nothing; the third uses keys 9..14
    ref, _ = attention_lse(q[None, 7:15], k[None, 9:15], v[None, 9:15], [6])
    assert np.allclose(out[7:15], ref[0], rtol=1e-12, atol=1e-13)


def test_merge_is_stable_for_far_apart_parts():
    # log-sum-exps 1500 apart: the part with the smaller one has weight exp(-1500) = 0
    r = rng(10)
    a, b = r.standard_normal((2, 1, 3, 24, D))
    la = np.full((1, 24, 3), 2000.0)
    lb = np.full((1, 24, 3), 500.0)
    out, l = merge_partials([a, b], [la, lb])
    assert np.isfinite(out).all() and np.isfinite(l).all()
    assert np.allclose(out, a, rtol=1e-14, atol=0) and np.allclose(l, 2000.0, rtol=1e-15, atol=0)
