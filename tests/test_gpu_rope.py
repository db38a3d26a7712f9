"""GPU parity of hv_rope3d_apply against the fp64 oracle (through the C ABI).

Small grids are compared on every element; the five benchmark workloads on
sampled rows.  Gate per element: within one bf16 spacing of the fp64 value plus 1e-4
(the kernel rotates in fp32 and rounds once), plus the workload's max-abs /
mean-abs gates.  Text rows must be bit-identical before and after.
"""
import numpy as np
import pytest

import hvinputs
from hvtest_util import bf16_ulp, bits_to_torch, log, torch_to_bits, widen
from oracle import apply_rope3d, token_grid

pytestmark = pytest.mark.gpu


def run_rope(bits_q, bits_k, F, H, W, theta, strided=False):
    import torch
    import rope_joint_attention_amd as hv

    g = hv.hv_token_grid(F, H, W)
    if strided:
        # q and k as views of one fused [B, L, 3, 24, 128] buffer
        B, L = bits_q.shape[:2]
        fused = torch.zeros((B, L, 3, 24, 128), dtype=torch.bfloat16, device="cuda")
        fused[:, :, 0] = bits_to_torch(bits_q)
        fused[:, :, 1] = bits_to_torch(bits_k)
        q, k = fused[:, :, 0], fused[:, :, 1]
    else:
        q, k = bits_to_torch(bits_q), bits_to_torch(bits_k)
    hv.hv_rope3d_apply(q, k, g, theta)
    torch.cuda.synchronize()
    return g, torch_to_bits(q), torch_to_bits(k)


def check(bits_in, bits_out, grid, theta, rows=None):
    L = bits_in.shape[1]
    if rows is None:
        rows = np.arange(L)
    ref = apply_rope3d(widen(bits_in[:, rows]), rows, grid, theta)
    got = widen(bits_out[:, rows])
    err = np.abs(got - ref)
    # one rounding of an fp32 rotation: at most one bf16 spacing away, plus the
    # fp32 angle error (pos * freq rounded in fp32: <= 79 * 2^-24 rad, times |x|)
    assert np.all(err <= bf16_ulp(ref) + 1e-4), float((err - bf16_ulp(ref)).max())
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    text = rows >= grid.n_video
    assert np.array_equal(bits_out[:, rows[text]], bits_in[:, rows[text]])
    return float(err.max()), float(err.mean())


@pytest.mark.parametrize("F,H,W,text,batch,theta,strided", [
    (1, 16, 16, 3, 1, 10000.0, False),     # 1 video token
    (5, 48, 80, 20, 2, 10000.0, False),    # 2 x 3 x 5, ragged
    (9, 64, 112, 0, 1, 256.0, False),      # no text rows, theta from the notes page
    (13, 96, 160, 37, 3, 10000.0, True),   # fused qkv strides
    (1, 256, 256, 256, 1, 10000.0, False), # image workload shape
])
def test_rope_small(F, H, W, text, batch, theta, strided):
    g = token_grid(F, H, W)
    L = g.n_video + text
    bits = hvinputs.draw_qkv(batch, L, seed=F * 131 + H + W)
    log(f"rope small F={F} H={H} W={W} L={L} B={batch} theta={theta} strided={strided}")
    _, q2, k2 = run_rope(bits["q"], bits["k"], F, H, W, theta, strided)
    check(bits["q"], q2, g, theta)
    check(bits["k"], k2, g, theta)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", hvinputs.WORKLOAD_ORDER)
def test_rope_workloads(name):
    wl = hvinputs.WORKLOADS[name]
    g = token_grid(wl.frames, wl.height, wl.width)
    L = g.n_video + wl.text_capacity
    log(f"rope workload {name} B={wl.batch} L={L}")
    bits = hvinputs.draw_qkv(wl.batch, L, wl.seed)
    _, q2, k2 = run_rope(bits["q"], bits["k"], wl.frames, wl.height, wl.width, wl.theta)
    rows = hvinputs.sample_rows(L, g.n_video, g.gh * g.gw, wl.seed, n_random=128, edge=32)
    mq = check(bits["q"], q2, g, wl.theta, rows)
    mk = check(bits["k"], k2, g, wl.theta, rows)
    log(f"  max/mean abs q={mq} k={mk}")
    # text rows bit-identical everywhere, not just on sampled rows
    assert np.array_equal(q2[:, g.n_video:], bits["q"][:, g.n_video:])
    assert np.array_equal(k2[:, g.n_video:], bits["k"][:, g.n_video:])


def test_rope_twice_equals_composition_within_rounding():
    # applying the call twice rotates by twice the angle (R(p)R(p) = R(2p)),
    # up to two bf16 roundings
    g = token_grid(5, 32, 48)
    L = g.n_video + 4
    bits = hvinputs.draw_qkv(1, L, seed=5)
    _, q1, k1 = run_rope(bits["q"], bits["k"], 5, 32, 48, 10000.0)
    _, q2, _ = run_rope(q1, k1, 5, 32, 48, 10000.0)
    once = apply_rope3d(widen(bits["q"]), np.arange(L), g, 10000.0)
    twice = apply_rope3d(once, np.arange(L), g, 10000.0)
    err = np.abs(widen(q2) - twice)
    # the first rounding error is rotated by the second call, so bound by the
    # spacing at the pair's norm rather than at each component
    pair_norm = np.sqrt(twice[..., 0::2] ** 2 + twice[..., 1::2] ** 2)
    bound = np.repeat(2.0 * bf16_ulp(pair_norm), 2, axis=-1) + 2e-4
    assert np.all(err <= bound)
