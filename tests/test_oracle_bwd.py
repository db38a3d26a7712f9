"""Pins of the fp64 oracle's attention gradients (joint_attention_bwd).

No page prints a gradient.  The pins tie the analytic gradients to the
already-pinned forward: central finite differences of the scalar
sum(dO * O) computed with joint_attention, plus identities any correct
gradient obeys (padded keys get nothing; shifting every key by one vector
leaves O unchanged, so the key gradients sum to zero; each softmax row sums
to one, so the value gradients sum to the summed output gradient; equal keys
give a zero query gradient).
"""
import math

import numpy as np
import pytest

from oracle import joint_attention, joint_attention_bwd

D = 128


def setup(seed, B=1, L=9, H=2, N=6, valid=(2,), qs=1.0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, L, H, D)) * qs
    k = r.standard_normal((B, L, H, D))
    v = r.standard_normal((B, L, H, D))
    g = r.standard_normal((B, L, H, D))
    return q, k, v, g, N, list(valid)


def loss(q, k, v, g, N, valid, scale=None):
    return float(np.sum(g * joint_attention(q, k, v, N, valid, scale=scale)))


@pytest.mark.parametrize("seed,qs,scale", [(1, 1.0, None), (2, 3.0, None), (3, 1.0, 0.3)])
def test_finite_differences(seed, qs, scale):
    q, k, v, g, N, valid = setup(seed, B=2, valid=(2, 3), qs=qs)
    dq, dk, dv = joint_attention_bwd(q, k, v, g, N, valid, scale=scale)
    r = np.random.default_rng(seed + 100)
    eps = 1e-6
    for name, t, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = tuple(int(r.integers(0, n)) for n in t.shape)
            if name != "q" and idx[1] >= N + valid[idx[0]]:
                continue   # padded keys are checked separately
            old = t[idx]
            t[idx] = old + eps
            lp = loss(q, k, v, g, N, valid, scale)
            t[idx] = old - eps
            lm = loss(q, k, v, g, N, valid, scale)
            t[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_padded_keys_get_no_gradient():
    q, k, v, g, N, valid = setup(4, B=2, valid=(0, 3))
    dq, dk, dv = joint_attention_bwd(q, k, v, g, N, valid)
    for b in range(2):
        n = N + valid[b]
        assert not dk[b, n:].any() and not dv[b, n:].any()
        assert np.abs(dk[b, :n]).max() > 0 and np.abs(dv[b, :n]).max() > 0
    # and poisoning them changes nothing anywhere
    k2, v2 = k.copy(), v.copy()
    k2[0, N:] = np.nan
    v2[1, N + 3:] = 1e30
    dq2, dk2, dv2 = joint_attention_bwd(q, k2, v2, g, N, valid)
    assert np.array_equal(dq2, dq)


def test_key_gradients_sum_to_zero_and_value_gradients_sum_to_dout():
    q, k, v, g, N, valid = setup(5, B=2, L=20, N=15, valid=(5, 1))
    dq, dk, dv = joint_attention_bwd(q, k, v, g, N, valid)
    for b in range(2):
        assert np.allclose(dk[b].sum(axis=0), 0.0, atol=1e-12)
        assert np.allclose(dv[b].sum(axis=0), g[b].sum(axis=0), rtol=1e-12, atol=1e-12)


def test_equal_keys_give_zero_query_gradient_and_mean_value_gradient():
    q, k, v, g, N, valid = setup(6, L=12, N=12, valid=(0,))
    k[:] = k[:, :1]
    dq, dk, dv = joint_attention_bwd(q, k, v, g, N, valid)
    assert np.allclose(dq, 0.0, atol=1e-12)
    # uniform weights: dV_j = mean over queries of dO, for every key
    assert np.allclose(dv[0], g[0].sum(axis=0, keepdims=True) / 12, rtol=1e-12, atol=1e-13)


def test_value_gradient_does_not_depend_on_values():
    q, k, v, g, N, valid = setup(7)
    _, _, dv1 = joint_attention_bwd(q, k, v, g, N, valid)
    _, _, dv2 = joint_attention_bwd(q, k, 5.0 * v + 1.0, g, N, valid)
    assert np.array_equal(dv1, dv2)


def test_one_key_closed_form():
    # a single key: P = 1, so dV = sum of dO, dS = 0, dQ = dK = 0
    q, k, v, g, N, valid = setup(8, L=5, N=1, valid=(0,))
    dq, dk, dv = joint_attention_bwd(q, k, v, g, N, valid)
    assert np.allclose(dq, 0, atol=1e-13) and np.allclose(dk, 0, atol=1e-13)
    assert np.allclose(dv[0, 0], g[0].sum(axis=0), rtol=1e-13, atol=1e-13)
    assert not dv[0, 1:].any()


def test_dq_rows_matches_the_full_gradient():
    from oracle import joint_attention_bwd_dq_rows

    q, k, v, g, N, valid = setup(9, B=2, L=14, N=10, valid=(1, 4))
    dq, _, _ = joint_attention_bwd(q, k, v, g, N, valid)
    rows = np.array([0, 3, 10, 13])
    sub = joint_attention_bwd_dq_rows(q[:, rows], k, v, g[:, rows], N, valid)
    assert np.allclose(sub, dq[:, rows], rtol=1e-13, atol=1e-14)


def test_varlen_bwd_finite_differences_and_isolation():
    from oracle import varlen_attention, varlen_attention_bwd

    r = np.random.default_rng(11)
    T, H = 17, 2
    q, k, v, g = (r.standard_normal((T, H, D)) for _ in range(4))
    cu_q, cu_k = [0, 6, 6, 15], [0, 4, 9, 16]   # an empty query segment; row 15, 16 outside
    dq, dk, dv = varlen_attention_bwd(q, k, v, g, cu_q, cu_k)

    def lossf():
        out, _ = varlen_attention(q, k, v, cu_q, cu_k)
        return float(np.sum(g * out))

    eps = 1e-6
    for name, t, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(10):
            idx = tuple(int(r.integers(0, n)) for n in t.shape)
            old = t[idx]
            t[idx] = old + eps
            lp = lossf()
            t[idx] = old - eps
            lm = lossf()
            t[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
    # keys 4..8 belong to the empty query segment: nobody attends to them
    assert not dk[4:9].any() and not dv[4:9].any()
    assert not dq[15:].any() and not dk[16:].any()


def test_varlen_bwd_matches_per_clip_joint_gradients():
    from oracle import varlen_attention_bwd

    r = np.random.default_rng(12)
    lens = [7, 12, 5]
    T = sum(lens)
    q, k, v, g = (r.standard_normal((T, 3, D)) for _ in range(4))
    cu = np.concatenate([[0], np.cumsum(lens)])
    dq, dk, dv = varlen_attention_bwd(q, k, v, g, cu, cu)
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        ref = joint_attention_bwd(q[None, a:b], k[None, a:b], v[None, a:b], g[None, a:b], b - a, [0])
        for got, want in zip((dq, dk, dv), ref):
            assert np.allclose(got[a:b], want[0], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("chunk,workers", [(1, 1), (3, 1), (7, 4), (256, 1)])
def test_by_rows_matches_the_full_gradient(chunk, workers):
    # the query-chunked form must equal the one-matrix form for every chunk
    # size, ragged last chunks included, on selected batch entries and heads
    from oracle import joint_attention_bwd_by_rows

    q, k, v, g, N, valid = setup(13, B=3, L=23, H=3, N=17, valid=(6, 0, 4), qs=2.0)
    ref = joint_attention_bwd(q, k, v, g, N, valid, heads=[2, 0])
    got = joint_attention_bwd_by_rows(q, k, v, g, N, valid, heads=[2, 0], batches=[2, 0],
                                      chunk=chunk, workers=workers)
    for want, have in zip(ref, got):
        assert np.allclose(have, want[[2, 0]], rtol=1e-12, atol=1e-13)


def test_by_rows_finite_differences_sums_and_padding():
    from oracle import joint_attention_bwd_by_rows

    q, k, v, g, N, valid = setup(14, B=2, L=11, N=8, valid=(3, 1), qs=1.5)
    dq, dk, dv = joint_attention_bwd_by_rows(q, k, v, g, N, valid, chunk=4)
    r = np.random.default_rng(15)
    eps = 1e-6
    for name, t, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(10):
            idx = tuple(int(r.integers(0, n)) for n in t.shape)
            if name != "q" and idx[1] >= N + valid[idx[0]]:
                continue
            old = t[idx]
            t[idx] = old + eps
            lp = loss(q, k, v, g, N, valid)
            t[idx] = old - eps
            lm = loss(q, k, v, g, N, valid)
            t[idx] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
    for b in range(2):
        n = N + valid[b]
        assert not dk[b, n:].any() and not dv[b, n:].any()
        assert np.allclose(dk[b].sum(axis=0), 0.0, atol=1e-12)
        assert np.allclose(dv[b].sum(axis=0), g[b].sum(axis=0), rtol=1e-12, atol=1e-12)
