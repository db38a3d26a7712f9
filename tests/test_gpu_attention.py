"""GPU parity of hv_joint_attention_fwd (and the full hot path) against the
fp64 oracle, through the C ABI.

* small shapes around the tile sizes (64-key tiles, 256-row query blocks),
  ragged tails, text-only and single-key sequences, batch > 1 with different
  valid text lengths: every output element;
* the five benchmark workloads end to end (token grid -> RoPE -> attention)
  against the oracle's hot path, and attention alone against the oracle run
  on the GPU's own rotated bf16 Q/K: all rows for the image workload,
  sampled rows for the others (every text row, the first and last 128 video
  rows, both rows at every frame boundary, 1024 seeded random rows);
* stress and edge cases: peaky softmax (Q x 8), identical keys (mean of V),
  theta = 256, NaN/huge values in padded K/V rows, determinism, every output
  row written (NaN-prefilled output), no writes outside the output rows
  (guard rows around a strided view), q, k, v and out as views of fused
  [B, L, 3, 24, 128] buffers (token stride of three head rows) giving the
  bits of contiguous tensors, for both block sizes.
"""
import numpy as np
import pytest

import hvinputs
from hvtest_util import assert_close, bits_to_torch, errors, log, torch_to_bits, widen
from oracle import apply_rope3d, hot_path, joint_attention, token_grid

pytestmark = pytest.mark.gpu


def gpu_attention(qb, kb, vb, n_video, valid, scale=None):
    import torch
    import rope_joint_attention_amd as hv

    q, k, v = bits_to_torch(qb), bits_to_torch(kb), bits_to_torch(vb)
    out = hv.hv_joint_attention_fwd(q, k, v, valid, n_video, softmax_scale=scale)
    torch.cuda.synchronize()
    return torch_to_bits(out)


SMALL = [
    # batch, n_video, text capacity, valid text per batch entry
    (1, 1, 0, [0]),            # one token
    (1, 0, 5, [5]),            # text only
    (1, 3, 4, [0]),            # all text padded
    (1, 40, 24, [10]),         # L = 64
    (2, 63, 2, [0, 2]),        # L = 65, keys 63 and 65
    (1, 200, 56, [56]),        # L = 256, one full query block
    (1, 200, 57, [13]),        # L = 257
    (2, 300, 45, [45, 3]),
    (1, 900, 124, [100]),      # L = 1024
    (3, 1500, 37, [37, 0, 20]),
    (1, 2047, 256, [255]),
    (64, 60, 10, [i % 11 for i in range(64)]),   # maximum batch, every valid length 0..10
]


@pytest.mark.parametrize("B,n_video,cap,valid", SMALL, ids=lambda x: str(x))
def test_attention_small(B, n_video, cap, valid):
    L = n_video + cap
    bits = hvinputs.draw_qkv(B, L, seed=7 * L + B)
    log(f"attention small B={B} N={n_video} L={L} valid={valid}")
    got = widen(gpu_attention(bits["q"], bits["k"], bits["v"], n_video, valid))
    ref = joint_attention(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), n_video, valid)
    e = assert_close(got, ref, f"B={B} N={n_video} L={L}")
    log(f"  {e}")


def test_attention_default_valid_is_all_text():
    B, n_video, cap = 2, 100, 30
    bits = hvinputs.draw_qkv(B, n_video + cap, seed=3)
    a = gpu_attention(bits["q"], bits["k"], bits["v"], n_video, None)
    b = gpu_attention(bits["q"], bits["k"], bits["v"], n_video, [cap, cap])
    assert np.array_equal(a, b)


def test_attention_explicit_scale():
    bits = hvinputs.draw_qkv(1, 300, seed=4)
    got = widen(gpu_attention(bits["q"], bits["k"], bits["v"], 250, [50], scale=0.3))
    ref = joint_attention(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), 250, [50], scale=0.3)
    assert_close(got, ref, "scale 0.3")


@pytest.mark.parametrize("q_scale", [4.0, 8.0])
def test_attention_peaky_softmax(q_scale):
    # large logits: the running reference must be raised many times
    B, n_video, cap, valid = 1, 1800, 200, [150]
    bits = hvinputs.draw_qkv(B, n_video + cap, seed=11, q_scale=q_scale)
    got = widen(gpu_attention(bits["q"], bits["k"], bits["v"], n_video, valid))
    ref = joint_attention(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), n_video, valid)
    e = assert_close(got, ref, f"q x {q_scale}")
    log(f"  peaky x{q_scale}: {e}")


def _directed_inputs(L, seed, key_boost):
    """q rows near 10 u for a fixed unit vector u, k rows with key_boost[j] u
    added: scores grow (or jump) along the sequence as key_boost says."""
    r = np.random.default_rng(seed)
    u = r.standard_normal(128)
    u /= np.linalg.norm(u)
    q = 0.3 * r.standard_normal((1, L, 24, 128)) + 10.0 * u
    k = r.standard_normal((1, L, 24, 128)) + key_boost[None, :, None, None] * u
    v = r.standard_normal((1, L, 24, 128))
    return {n: hvinputs.f32_to_bf16_bits(x.astype(np.float32)) for n, x in (("q", q), ("k", k), ("v", v))}


@pytest.mark.parametrize("case", ["rising", "late_jump"])
def test_attention_weight_bounds(case):
    """Scores that rise along the sequence by ~80 (log2 units): the sum of
    weights passes 2^40 and the reference moves up in steps of 32; and scores
    that jump by ~150 in a late tile, past the fp32 range of the first
    tile's reference, so the block is redone with per-tile maxima.  Both
    paths (packed V and V in place) must agree bit for bit and match the
    oracle."""
    import torch
    import rope_joint_attention_amd as hv

    n_video, cap, valid = 2300, 20, [20]
    L = n_video + cap
    boost = np.zeros(L)
    if case == "rising":
        boost[:] = np.linspace(0.0, 60.0, L)
    else:
        boost[2200:2240] = 110.0
    bits = _directed_inputs(L, 99, boost)
    q, k, v = (bits_to_torch(bits[n]) for n in ("q", "k", "v"))
    a = hv.hv_joint_attention_fwd(q, k, v, valid, n_video)
    b = hv.hv_joint_attention_fwd(q, k, v, valid, n_video, pack_v=False)
    torch.cuda.synchronize()
    a, b = torch_to_bits(a), torch_to_bits(b)
    assert np.array_equal(a, b)
    ref = joint_attention(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), n_video, valid)
    e = assert_close(widen(a), ref, case)
    log(f"  {case}: {e}")


def test_attention_identical_keys_give_mean_of_v():
    B, n_video, cap, valid = 1, 700, 60, [33]
    L = n_video + cap
    bits = hvinputs.draw_qkv(B, L, seed=12)
    k = np.broadcast_to(bits["k"][:, :1], bits["k"].shape).copy()
    got = widen(gpu_attention(bits["q"], k, bits["v"], n_video, valid))
    mean = widen(bits["v"])[0, :n_video + valid[0]].mean(axis=0)
    assert_close(got[0], np.broadcast_to(mean, got[0].shape), "mean of V", rel_fro=2e-2)


def test_attention_poisoned_padding_is_ignored():
    B, n_video, cap, valid = 2, 500, 100, [7, 0]
    L = n_video + cap
    bits = hvinputs.draw_qkv(B, L, seed=13)
    clean = gpu_attention(bits["q"], bits["k"], bits["v"], n_video, valid)
    k, v = bits["k"].copy(), bits["v"].copy()
    for b in range(B):
        lk = n_video + valid[b]
        k[b, lk:] = 0x7FC0   # NaN
        v[b, lk:] = 0x7F7F   # ~3.4e38
    dirty = gpu_attention(bits["q"], k, v, n_video, valid)
    assert np.array_equal(clean, dirty)
    ref = joint_attention(widen(bits["q"]), widen(k), widen(v), n_video, valid)
    assert_close(widen(dirty), ref, "poisoned padding")


def test_attention_deterministic_and_fully_written():
    import torch
    import rope_joint_attention_amd as hv

    B, n_video, cap = 2, 1000, 77
    L = n_video + cap
    bits = hvinputs.draw_qkv(B, L, seed=14)
    q, k, v = (bits_to_torch(bits[n]) for n in ("q", "k", "v"))
    outs = []
    for _ in range(3):
        out = torch.full_like(q, float("nan"))
        hv.hv_joint_attention_fwd(q, k, v, [77, 5], n_video, out=out)
        torch.cuda.synchronize()
        outs.append(torch_to_bits(out))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    assert np.all(np.isfinite(widen(outs[0])))


@pytest.mark.parametrize("B,n_video,cap,valid", [
    (1, 400, 50, [31]),          # 4-wave blocks, V in place
    (2, 1300, 100, [100, 7]),    # 288 blocks of 256 rows: packed V, persistent workgroups
])
def test_attention_fused_qkv_views(B, n_video, cap, valid):
    """q, k, v (and out) as views of fused [B, L, 3, 24, 128] buffers, so the
    token stride is three head rows: the same bits as contiguous tensors."""
    import torch
    import rope_joint_attention_amd as hv

    L = n_video + cap
    bits = hvinputs.draw_qkv(B, L, seed=3 * L + B)
    fused = torch.zeros((B, L, 3, 24, 128), dtype=torch.bfloat16, device="cuda")
    for i, n in enumerate("qkv"):
        fused[:, :, i] = bits_to_torch(bits[n])
    out_f = torch.full((B, L, 3, 24, 128), 5.0, dtype=torch.bfloat16, device="cuda")
    log(f"fused qkv views B={B} L={L} valid={valid}")
    hv.hv_joint_attention_fwd(fused[:, :, 0], fused[:, :, 1], fused[:, :, 2], valid, n_video,
                              out=out_f[:, :, 1])
    flat = hv.hv_joint_attention_fwd(*(bits_to_torch(bits[n]) for n in "qkv"), valid, n_video)
    torch.cuda.synchronize()
    assert torch.all(out_f[:, :, 0] == 5.0) and torch.all(out_f[:, :, 2] == 5.0)
    got = torch_to_bits(out_f[:, :, 1].contiguous())
    assert np.array_equal(got, torch_to_bits(flat))
    if B * L <= 1000:
        ref = joint_attention(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), n_video, valid)
        assert_close(widen(got), ref, "fused qkv views")


def test_attention_guard_rows_untouched():
    """Strided views with one guard row before and after every sequence."""
    import torch
    import rope_joint_attention_amd as hv

    B, n_video, cap, valid = 2, 300, 40, [40, 11]
    L = n_video + cap
    bits = hvinputs.draw_qkv(B, L, seed=15)

    def framed(x):
        buf = torch.full((B, L + 2, 24, 128), 7.0, dtype=torch.bfloat16, device="cuda")
        buf[:, 1:L + 1] = bits_to_torch(x)
        return buf

    qb, kb, vb = framed(bits["q"]), framed(bits["k"]), framed(bits["v"])
    ob = torch.full((B, L + 2, 24, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    hv.hv_joint_attention_fwd(qb[:, 1:L + 1], kb[:, 1:L + 1], vb[:, 1:L + 1], valid, n_video,
                              out=ob[:, 1:L + 1])
    torch.cuda.synchronize()
    assert torch.all(ob[:, 0] == 3.0) and torch.all(ob[:, L + 1] == 3.0)
    got = widen(torch_to_bits(ob[:, 1:L + 1]))
    ref = joint_attention(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), n_video, valid)
    assert_close(got, ref, "strided with guard rows")


def test_hot_path_theta_256():
    import torch
    import rope_joint_attention_amd as hv

    F, H, W, cap, valid = 9, 96, 128, 30, [17]
    g = hv.hv_token_grid(F, H, W)
    L = g.n_video + cap
    bits = hvinputs.draw_qkv(1, L, seed=16)
    q, k, v = (bits_to_torch(bits[n]) for n in ("q", "k", "v"))
    hv.hv_rope3d_apply(q, k, g, 256.0)
    out = hv.hv_joint_attention_fwd(q, k, v, valid, g.n_video)
    torch.cuda.synchronize()
    _, ref = hot_path(bits["q"], bits["k"], bits["v"], F, H, W, valid, 256.0)
    assert_close(widen(torch_to_bits(out)), ref, "theta 256 end to end")


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", hvinputs.WORKLOAD_ORDER)
def test_workload_end_to_end(name):
    """Full-size workload: GPU token grid -> RoPE -> attention vs the oracle."""
    import torch
    import rope_joint_attention_amd as hv

    wl = hvinputs.WORKLOADS[name]
    g = hv.hv_token_grid(wl.frames, wl.height, wl.width)
    og = token_grid(wl.frames, wl.height, wl.width)
    assert g.n_video == og.n_video
    L = g.n_video + wl.text_capacity
    log(f"workload {name}: B={wl.batch} L={L} valid={wl.valid}")
    bits = hvinputs.draw_qkv(wl.batch, L, wl.seed)
    q, k, v = (bits_to_torch(bits[n]) for n in ("q", "k", "v"))
    hv.hv_rope3d_apply(q, k, g, wl.theta)
    out = hv.hv_joint_attention_fwd(q, k, v, list(wl.valid), g.n_video)
    torch.cuda.synchronize()
    if name == "image_256x256":
        rows = np.arange(L)
    else:
        rows = hvinputs.sample_rows(L, g.n_video, g.gh * g.gw, wl.seed, n_random=1024, edge=128)
    got = widen(torch_to_bits(out)[:, rows])
    q_rot, k_rot = torch_to_bits(q), torch_to_bits(k)
    del q, k, v, out
    torch.cuda.empty_cache()

    # attention alone, on the GPU's own rotated bf16 Q/K
    ref_alone = joint_attention(widen(q_rot[:, rows]), widen(k_rot), widen(bits["v"]),
                                g.n_video, wl.valid)
    e1 = assert_close(got, ref_alone, f"{name} attention alone")
    log(f"  attention alone: {e1}")
    del k_rot
    # end to end against the oracle's fp64 RoPE of the original inputs
    _, ref = hot_path(bits["q"], bits["k"], bits["v"], wl.frames, wl.height, wl.width,
                      wl.valid, wl.theta, rows=rows)
    e2 = assert_close(got, ref, f"{name} end to end")
    log(f"  end to end: {e2}")
    # padded text rows versus valid rows (both computed over the same keys)
    for b in range(wl.batch):
        pad = rows >= g.n_video + wl.valid[b]
        if pad.any():
            log(f"  b={b} padded rows: {errors(got[b, pad], ref[b, pad])}")
