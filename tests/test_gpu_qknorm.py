"""GPU parity of hv_qk_norm_rope3d_apply (per-head RMSNorm, then 3D RoPE) against
the fp64 oracle, through the C ABI.

Gate per element: within one bf16 spacing of the fp64 value plus 2e-4 (the
kernel normalises and rotates in fp32 and rounds once; the extra term covers
the fp32 angle, rsqrt and sum-of-squares rounding at |y| up to ~10), plus the
workload's max-abs / mean-abs gates.  Small grids are compared on every
element, the five benchmark workloads on sampled rows (every text row
included) plus a full-tensor pair-magnitude property.
"""
import numpy as np
import pytest

import hvinputs
from hvtest_util import assert_close, bf16_ulp, bits_to_torch, log, torch_to_bits, widen
from oracle import joint_attention, qk_norm_rope3d, token_grid

pytestmark = pytest.mark.gpu


def scaled_bits(bits, factor_pow2):
    """Multiply bf16 bit patterns by 2**factor_pow2 exactly (exponent shift)."""
    f = widen(bits) * (2.0 ** factor_pow2)
    return hvinputs.f32_to_bf16_bits(f.astype(np.float32))


def run_qknorm(bits_q, bits_k, F, H, W, theta, gam, eps, text_gamma=True, strided=False):
    import torch
    import rope_joint_attention_amd as hv

    g = hv.hv_token_grid(F, H, W)
    if strided:
        B, L = bits_q.shape[:2]
        fused = torch.zeros((B, L, 3, 24, 128), dtype=torch.bfloat16, device="cuda")
        fused[:, :, 0] = bits_to_torch(bits_q)
        fused[:, :, 1] = bits_to_torch(bits_k)
        q, k = fused[:, :, 0], fused[:, :, 1]
    else:
        q, k = bits_to_torch(bits_q), bits_to_torch(bits_k)
    gt = {n: bits_to_torch(v) for n, v in gam.items()}
    hv.hv_qk_norm_rope3d_apply(q, k, g, theta, gt["q_video"], gt["k_video"],
                               gt["q_text"] if text_gamma else None,
                               gt["k_text"] if text_gamma else None, eps)
    torch.cuda.synchronize()
    return g, torch_to_bits(q), torch_to_bits(k)


def reference(bits_in, grid, theta, gv, gt, eps, rows):
    return qk_norm_rope3d(widen(bits_in[:, rows]), rows, grid, theta, widen(gv),
                          None if gt is None else widen(gt), eps)


def check(bits_in, bits_out, grid, theta, gv, gt, eps, rows=None):
    L = bits_in.shape[1]
    if rows is None:
        rows = np.arange(L)
    ref = reference(bits_in, grid, theta, gv, gt, eps, rows)
    got = widen(bits_out[:, rows])
    err = np.abs(got - ref)
    excess = err - (bf16_ulp(ref) + 2e-4)
    assert np.all(excess <= 0), float(excess.max())
    assert err.max() <= 2e-2 * max(1.0, np.abs(ref).max() / 4) and err.mean() <= 2e-3
    return float(err.max()), float(err.mean())


@pytest.mark.parametrize("F,H,W,text,batch,theta,eps,pow2,text_gamma,strided", [
    (1, 16, 16, 3, 1, 10000.0, 1e-6, 0, True, False),     # 1 video token
    (5, 48, 80, 20, 2, 10000.0, 1e-6, 3, True, False),    # 2 x 3 x 5, ragged, inputs x8
    (9, 64, 112, 0, 1, 256.0, 1e-5, -4, False, False),    # no text rows, shared weights
    (13, 96, 160, 37, 3, 10000.0, 1e-6, 0, True, True),   # fused qkv strides
    (1, 256, 256, 256, 1, 10000.0, 1e-6, 6, True, False), # image workload shape, inputs x64
    (5, 32, 48, 11, 1, 10000.0, 0.0, 0, True, False),     # eps = 0
])
def test_qknorm_small(F, H, W, text, batch, theta, eps, pow2, text_gamma, strided):
    g = token_grid(F, H, W)
    L = g.n_video + text
    bits = hvinputs.draw_qkv(batch, L, seed=F * 977 + H + W)
    bq, bk = scaled_bits(bits["q"], pow2), scaled_bits(bits["k"], pow2)
    gam = hvinputs.draw_gamma(seed=F + H + W)
    log(f"qknorm small F={F} H={H} W={W} L={L} B={batch} eps={eps} x2^{pow2} text_gamma={text_gamma}")
    _, q2, k2 = run_qknorm(bq, bk, F, H, W, theta, gam, eps, text_gamma, strided)
    check(bq, q2, g, theta, gam["q_video"], gam["q_text"] if text_gamma else None, eps)
    check(bk, k2, g, theta, gam["k_video"], gam["k_text"] if text_gamma else None, eps)


def test_qknorm_tiny_inputs_where_eps_matters():
    # |x| ~ 2^-12: mean(x^2) ~ 6e-8 is comparable to eps = 1e-7, so a misplaced eps shows
    g = token_grid(5, 32, 48)
    L = g.n_video + 9
    bits = hvinputs.draw_qkv(1, L, seed=77)
    bq, bk = scaled_bits(bits["q"], -12), scaled_bits(bits["k"], -12)
    gam = hvinputs.draw_gamma(seed=78)
    _, q2, k2 = run_qknorm(bq, bk, 5, 32, 48, 10000.0, gam, 1e-7)
    check(bq, q2, g, 10000.0, gam["q_video"], gam["q_text"], 1e-7)
    check(bk, k2, g, 10000.0, gam["k_video"], gam["k_text"], 1e-7)


def test_qknorm_zero_rows_give_zero_with_eps():
    g = token_grid(5, 32, 48)
    L = g.n_video + 4
    bits = hvinputs.draw_qkv(1, L, seed=79)
    bq = bits["q"].copy()
    bq[0, 3] = 0          # a zero video row
    bq[0, L - 1, 7] = 0   # one zero head of a text row
    gam = hvinputs.draw_gamma(seed=80)
    _, q2, _ = run_qknorm(bq, bits["k"], 5, 32, 48, 10000.0, gam, 1e-6)
    assert not np.any(widen(q2[0, 3])) and not np.any(widen(q2[0, L - 1, 7]))
    check(bq, q2, g, 10000.0, gam["q_video"], gam["q_text"], 1e-6)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", hvinputs.WORKLOAD_ORDER)
def test_qknorm_workloads(name):
    wl = hvinputs.WORKLOADS[name]
    g = token_grid(wl.frames, wl.height, wl.width)
    L = g.n_video + wl.text_capacity
    log(f"qknorm workload {name} B={wl.batch} L={L}")
    bits = hvinputs.draw_qkv(wl.batch, L, wl.seed)
    gam = hvinputs.draw_gamma(wl.seed)
    _, q2, k2 = run_qknorm(bits["q"], bits["k"], wl.frames, wl.height, wl.width, wl.theta, gam, 1e-6)
    rows = hvinputs.sample_rows(L, g.n_video, g.gh * g.gw, wl.seed, n_random=128, edge=32)
    mq = check(bits["q"], q2, g, wl.theta, gam["q_video"], gam["q_text"], 1e-6, rows)
    mk = check(bits["k"], k2, g, wl.theta, gam["k_video"], gam["k_text"], 1e-6, rows)
    log(f"  max/mean abs q={mq} k={mk}")
    # Every row of the full tensor, via a property that holds at any size: the
    # rotation keeps the magnitude of each channel pair, so pair (2j, 2j+1) of
    # the output has the magnitude of the same pair of gamma * x / rms(x), on
    # video rows (rotated) and text rows (not rotated) alike.  Catches rows left
    # unprocessed, a wrong weight stream and a wrong normaliser anywhere.
    for bits_in, bits_out, gv, gtx in ((bits["q"], q2, gam["q_video"], gam["q_text"]),
                                       (bits["k"], k2, gam["k_video"], gam["k_text"])):
        for b in range(wl.batch):
            x = widen(bits_in[b]).astype(np.float32)
            y = widen(bits_out[b]).astype(np.float32)
            gamma = np.where((np.arange(L) < g.n_video)[:, None], widen(gv)[None, :],
                             widen(gtx)[None, :]).astype(np.float32)[:, None, :]
            t = gamma * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + np.float32(1e-6))
            pt = np.sqrt(t[..., 0::2] ** 2 + t[..., 1::2] ** 2)
            py = np.sqrt(y[..., 0::2] ** 2 + y[..., 1::2] ** 2)
            # two bf16 roundings of a pair: at most one spacing at the pair norm, plus fp32 slack
            bound = 2.0 ** (np.floor(np.log2(np.maximum(pt, 2.0 ** -126))) - 7) + 1e-4
            bad = np.abs(py - pt) > bound
            assert not bad.any(), (b, int(bad.sum()), float(np.abs(py - pt).max()))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["image_256x256", "video_720x1280x33_b2"])
def test_qknorm_then_attention_end_to_end(name):
    # the prologue feeding the attention kernel, against the oracle's fp64
    # norm -> rope -> attention on the original bf16 inputs
    import torch
    import rope_joint_attention_amd as hv

    wl = hvinputs.WORKLOADS[name]
    g = token_grid(wl.frames, wl.height, wl.width)
    L = g.n_video + wl.text_capacity
    bits = hvinputs.draw_qkv(wl.batch, L, wl.seed)
    gam = hvinputs.draw_gamma(wl.seed)
    log(f"qknorm -> attention {name} B={wl.batch} L={L}")
    _, q2, k2 = run_qknorm(bits["q"], bits["k"], wl.frames, wl.height, wl.width, wl.theta, gam, 1e-6)
    out = hv.hv_joint_attention_fwd(bits_to_torch(q2), bits_to_torch(k2), bits_to_torch(bits["v"]),
                                    list(wl.valid), g.n_video)
    torch.cuda.synchronize()
    ob = torch_to_bits(out)
    rows = hvinputs.sample_rows(L, g.n_video, g.gh * g.gw, wl.seed, n_random=64, edge=16)
    if L <= 1024:
        rows = np.arange(L)
    qf = qk_norm_rope3d(widen(bits["q"][:, rows]), rows, g, wl.theta, widen(gam["q_video"]),
                        widen(gam["q_text"]), 1e-6)
    kf = qk_norm_rope3d(widen(bits["k"]), np.arange(L), g, wl.theta, widen(gam["k_video"]),
                        widen(gam["k_text"]), 1e-6)
    ref = joint_attention(qf, kf, widen(bits["v"]), g.n_video, wl.valid)
    e = assert_close(widen(ob[:, rows]), ref, f"{name} norm+rope+attention")
    log(f"  {e}")


def test_qknorm_maximum_batch():
    import rope_joint_attention_amd as hv

    g = token_grid(5, 32, 48)
    L = g.n_video + 3
    B = hv.HV_MAX_BATCH
    bits = hvinputs.draw_qkv(B, L, seed=646)
    gam = hvinputs.draw_gamma(seed=647)
    _, q2, k2 = run_qknorm(bits["q"], bits["k"], 5, 32, 48, 10000.0, gam, 1e-6)
    check(bits["q"], q2, g, 10000.0, gam["q_video"], gam["q_text"], 1e-6)
    check(bits["k"], k2, g, 10000.0, gam["k_video"], gam["k_text"], 1e-6)
