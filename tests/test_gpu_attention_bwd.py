"""GPU parity of hv_joint_attention_bwd (dQ, dK, dV) against the fp64 oracle,
through the C ABI.

The forward runs on the GPU first (hv_attention_fwd_lse gives out and the
log-sum-exp the backward consumes); the oracle computes the gradients from
the same bf16 q, k, v, dout in fp64.  Gates, per gradient: relative Frobenius
error <= 1e-2, max-abs error <= 2e-2 * max|ref|, mean-abs <= 2e-3 * max|ref|,
no NaN/Inf; the kernel rounds P and dS to bf16 as MFMA operands (2^-9
relative each, averaging out) and reads O in bf16, so a correct kernel sits
near 2e-3 relative.  Sizes are floored at 1e-3 per element, so an exactly-zero
reference gradient (a single key) is held to rounding noise below 2e-5.
Padded keys must get exactly zero dK, dV.  At the workload sizes whole heads
are compared on every row and key (the oracle's query-chunked gradients
never hold an L x L matrix).
"""
import numpy as np
import pytest

import hvinputs
from hvtest_util import bits_to_torch, log, torch_to_bits, widen
from oracle import joint_attention_bwd, joint_attention_bwd_dq_rows, token_grid

pytestmark = pytest.mark.gpu


def grad_close(got, ref, what, floor=1e-3):
    # errors are measured against the reference's size, but never against less
    # than `floor` per element: a gradient that is exactly zero (one key: dS = 0)
    # comes out of fp32 as rounding noise of the cancelling dP - D
    d = np.abs(got - ref)
    scale = max(float(np.abs(ref).max()), floor)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), floor * np.sqrt(ref.size)))
    e = {"rel_fro": rel, "max_rel": float(d.max()) / scale, "mean_rel": float(d.mean()) / scale}
    assert np.isfinite(got).all(), what
    assert rel <= 1e-2 and e["max_rel"] <= 2e-2 and e["mean_rel"] <= 2e-3, f"{what}: {e}"
    return e


def run_bwd(bits, dout_bits, n_video, valid, scale=None, fused=False):
    import torch
    import rope_joint_attention_amd as hv

    if fused:
        B, L = bits["q"].shape[:2]
        buf = torch.zeros((B, L, 3, 24, 128), dtype=torch.bfloat16, device="cuda")
        for i, n in enumerate("qkv"):
            buf[:, :, i] = bits_to_torch(bits[n])
        q, k, v = buf[:, :, 0], buf[:, :, 1], buf[:, :, 2]
    else:
        q, k, v = (bits_to_torch(bits[n]) for n in "qkv")
    lk = [n_video + x for x in valid]
    out, lse = hv.hv_attention_fwd_lse(q, k, v, lk, softmax_scale=scale)
    g = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    g.copy_(bits_to_torch(dout_bits))
    dq, dk, dv = hv.hv_joint_attention_bwd(q, k, v, out, g, lse, list(valid), n_video,
                                           softmax_scale=scale)
    torch.cuda.synchronize()
    return torch_to_bits(dq), torch_to_bits(dk), torch_to_bits(dv)


def draw(B, L, seed, q_scale=1.0):
    bits = hvinputs.draw_qkv(B, L, seed, q_scale=q_scale)
    dout = hvinputs.draw_qkv(B, L, seed + 7919)["q"]
    return bits, dout


@pytest.mark.parametrize("B,L,N,valid,scale,q_scale,fused", [
    (1, 1, 1, (0,), None, 1.0, False),
    (1, 40, 24, (10,), None, 1.0, False),
    (2, 129, 100, (29, 3), None, 1.0, False),
    (1, 300, 256, (44,), 0.05, 1.0, True),
    (3, 257, 200, (0, 57, 20), None, 4.0, False),   # peaky
    (1, 700, 640, (60,), None, 1.0, False),         # several tiles and key blocks, ragged
])
def test_bwd_small(B, L, N, valid, scale, q_scale, fused):
    bits, dout = draw(B, L, seed=L * 3 + N, q_scale=q_scale)
    log(f"bwd small B={B} L={L} N={N} valid={valid} scale={scale} q_scale={q_scale} fused={fused}")
    dq, dk, dv = run_bwd(bits, dout, N, valid, scale, fused)
    ref = joint_attention_bwd(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), widen(dout), N,
                              valid, scale=scale)
    for name, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        e = grad_close(widen(got), r, name)
        log(f"  {name} {e}")
    for b in range(B):
        n = N + valid[b]
        assert not widen(dk[b, n:]).any() and not widen(dv[b, n:]).any()


def test_bwd_poisoned_padding_and_determinism():
    import torch

    B, L, N, valid = 2, 200, 150, (20, 50)
    bits, dout = draw(B, L, seed=5)
    ref = run_bwd(bits, dout, N, valid)
    poisoned = {n: bits[n].copy() for n in "qkv"}
    nan = hvinputs.f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    poisoned["k"][0, N + 20:] = nan
    poisoned["v"][1, N + 50:] = nan
    again = run_bwd(poisoned, dout, N, valid)
    for a, b in zip(ref, again):
        assert np.array_equal(a, b)
    twice = run_bwd(bits, dout, N, valid)
    for a, b in zip(ref, twice):
        assert np.array_equal(a, b)


def test_bwd_workspace_holds_d_then_the_counters():
    # the delta workspace: -D = -rowsum(dO * O) per (batch, head, row) in fp32,
    # then -lse/scale in the same placement, then the work counters of the two
    # persistent gradient kernels (each ends at blocks + workgroups: every
    # workgroup's last take finds no block); the rest of the 256 counter bytes
    # is not written.  A second, smaller call reuses the workspace without
    # clearing it.
    import torch
    import rope_joint_attention_amd as hv

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    scale = 1.0 / np.sqrt(128.0)
    ws = torch.full((2 * 2 * 24 * 700 + hv.BWD_COUNTER_FLOATS,), 7.0, dtype=torch.float32, device="cuda")
    for B, L, N, valid, seed in ((2, 700, 640, (60, 13), 61), (1, 129, 100, (29,), 62)):
        bits, dout = draw(B, L, seed=seed)
        q, k, v = (bits_to_torch(bits[n]) for n in "qkv")
        g = bits_to_torch(dout)
        lk = [N + x for x in valid]
        out, lse = hv.hv_attention_fwd_lse(q, k, v, lk)
        log(f"bwd workspace B={B} L={L}")
        hv.hv_joint_attention_bwd(q, k, v, out, g, lse, list(valid), N, delta=ws)
        torch.cuda.synchronize()
        n = B * 24 * L
        d_ref = (out.float() * g.float()).sum(-1).permute(0, 2, 1).reshape(-1).cpu().numpy()
        got = ws.cpu().numpy()
        np.testing.assert_allclose(-got[:n], d_ref, rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(got[n:2 * n], -lse.cpu().numpy().reshape(-1) / scale, rtol=1e-6)
        cnt = got[2 * n:2 * n + 2].view(np.int32)
        kb, qb = B * 24 * ((L + 127) // 128), B * 24 * ((L + 255) // 256)
        assert cnt[0] == kb + min(kb, cus) and cnt[1] == qb + min(qb, cus), (cnt, kb, qb)
        if B == 2:
            assert (got[2 * n + 2:2 * n + hv.BWD_COUNTER_FLOATS] == 7.0).all()
            assert (got[2 * n + hv.BWD_COUNTER_FLOATS:] == 7.0).all()


@pytest.mark.timeout(600)
def test_bwd_image_workload_full():
    wl = hvinputs.WORKLOADS["image_256x256"]
    g = token_grid(wl.frames, wl.height, wl.width)
    L = g.n_video + wl.text_capacity
    bits, dout = draw(wl.batch, L, wl.seed)
    log(f"bwd image workload L={L}")
    dq, dk, dv = run_bwd(bits, dout, g.n_video, wl.valid)
    ref = joint_attention_bwd(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), widen(dout),
                              g.n_video, wl.valid)
    for name, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        log(f"  {name} {grad_close(widen(got), r, name)}")


# Heads (and batch entries) compared element by element on every row at the
# full workload sizes, with the query-chunked fp64 gradients of the oracle.
FULL_GRAD_HEADS = {
    "video_544x960x17": ([0, 13], [0]),
    "video_720x1280x33_b2": ([0, 13], [0, 1]),
    "video_544x960x129": ([5], [0]),
    "video_720x1280x129": ([17], [0]),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["video_544x960x17", "video_720x1280x33_b2", "video_544x960x129",
                                  "video_720x1280x129"])
def test_bwd_workloads(name):
    # dQ, dK and dV of the listed heads on every row and key against the
    # oracle; dQ of three heads on sampled rows; dK and dV of every head
    # through identities that hold at any size (the key gradients of each
    # (batch, head) sum to zero, the value gradients sum to the summed dO).
    import os

    from oracle import joint_attention_bwd_by_rows

    wl = hvinputs.WORKLOADS[name]
    g = token_grid(wl.frames, wl.height, wl.width)
    L = g.n_video + wl.text_capacity
    bits, dout = draw(wl.batch, L, wl.seed)
    log(f"bwd workload {name} B={wl.batch} L={L}")
    dq, dk, dv = run_bwd(bits, dout, g.n_video, wl.valid)
    rows = hvinputs.sample_rows(L, g.n_video, g.gh * g.gw, wl.seed, n_random=32, edge=8)
    heads = [0, 13, 23]
    ref = joint_attention_bwd_dq_rows(widen(bits["q"][:, rows]), widen(bits["k"]), widen(bits["v"]),
                                      widen(dout[:, rows]), g.n_video, wl.valid, heads=heads)
    log(f"  dq rows {grad_close(widen(dq[:, rows][:, :, heads]), ref, 'dq rows')}")
    del ref
    for b in range(wl.batch):
        n = g.n_video + wl.valid[b]
        dkb = widen(dk[b, :n]).sum(axis=0)              # [24, 128]
        scale_k = np.abs(widen(dk[b, :n])).sum(axis=0)
        assert np.all(np.abs(dkb) <= 2e-2 * scale_k + 1e-6), float((np.abs(dkb) / scale_k).max())
        dvb = widen(dv[b, :n]).sum(axis=0)
        gsum = widen(dout[b]).sum(axis=0)
        err = np.abs(dvb - gsum)
        assert np.all(err <= 1e-2 * np.abs(widen(dv[b, :n])).sum(axis=0) + 1e-3), float(err.max())
        assert not widen(dk[b, n:]).any() and not widen(dv[b, n:]).any()
    fh, fb = FULL_GRAD_HEADS[name]
    workers = max(1, min(16, os.cpu_count() or 1))
    for h in fh:
        sub = [t[:, :, h:h + 1] for t in (bits["q"], bits["k"], bits["v"], dout)]
        full = joint_attention_bwd_by_rows(*(widen(t) for t in sub), g.n_video, wl.valid,
                                           batches=fb, workers=workers)
        for i, (nm, got) in enumerate((("dq", dq), ("dk", dk), ("dv", dv))):
            e = grad_close(widen(got[fb][:, :, h:h + 1]), full[i], f"{nm} head {h}")
            log(f"  {nm} head {h} batch {fb} all rows {e}")


def test_bwd_maximum_batch():
    import rope_joint_attention_amd as hv

    B, L, N = hv.HV_MAX_BATCH, 48, 40
    valid = tuple(i % 9 for i in range(B))
    bits, dout = draw(B, L, seed=6400)
    log(f"bwd batch {B} L={L}")
    dq, dk, dv = run_bwd(bits, dout, N, valid)
    ref = joint_attention_bwd(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), widen(dout), N,
                              valid, heads=[0, 7, 23])
    for i, (name, got) in enumerate((("dq", dq), ("dk", dk), ("dv", dv))):
        grad_close(widen(got[:, :, [0, 7, 23]]), ref[i], name)


def run_varlen_bwd(bits, dout_bits, cq, ck):
    import torch
    import rope_joint_attention_amd as hv

    q, k, v = (bits_to_torch(bits[n])[0] for n in "qkv")
    out, lse = hv.hv_joint_attention_varlen_fwd(q, k, v, cq, ck, want_lse=True)
    g = bits_to_torch(dout_bits)[0]
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    hv.hv_joint_attention_varlen_bwd(q, k, v, out, g, lse, cq, ck, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return torch_to_bits(dq), torch_to_bits(dk), torch_to_bits(dv)


def test_varlen_bwd_packed_clips():
    from oracle import varlen_attention_bwd

    lens = [16 + 13, 30, 256 + 200, 24 + 77]   # clips [video | valid text] of the forward test
    cu = [0] + list(np.cumsum(lens))
    T = cu[-1]
    bits, dout = draw(1, T, seed=2121)
    log(f"varlen bwd clips T={T} cu={cu}")
    dq, dk, dv = run_varlen_bwd(bits, dout, cu, cu)
    ref = varlen_attention_bwd(widen(bits["q"][0]), widen(bits["k"][0]), widen(bits["v"][0]),
                               widen(dout[0]), cu, cu)
    for name, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        log(f"  {name} {grad_close(widen(got), r, name)}")


def test_varlen_bwd_cross_segments_and_untouched_rows():
    from oracle import varlen_attention_bwd

    T = 700
    bits, dout = draw(1, T, seed=3131)
    cq = [0, 100, 100, 400, 650]     # an empty query segment; rows 650.. belong to none
    ck = [0, 50, 60, 600, 690]       # keys 50..59 belong to the empty segment; 690.. to none
    dq, dk, dv = run_varlen_bwd(bits, dout, cq, ck)
    ref = varlen_attention_bwd(widen(bits["q"][0]), widen(bits["k"][0]), widen(bits["v"][0]),
                               widen(dout[0]), cq, ck)
    assert np.isnan(widen(dq[650:])).all()
    assert np.isnan(widen(dk[690:])).all() and np.isnan(widen(dv[690:])).all()
    assert not widen(dk[50:60]).any() and not widen(dv[50:60]).any()   # zero-filled
    grad_close(widen(dq[:650]), ref[0][:650], "dq")
    grad_close(widen(dk[:690]), ref[1][:690], "dk")
    grad_close(widen(dv[:690]), ref[2][:690], "dv")


def test_varlen_bwd_padded_batch_reading():
    # a padded batch of two entries flattened into [valid | padded tail]
    # segments, each tail attending to itself
    from oracle import varlen_attention_bwd

    B, N, cap, valid = 2, 600, 100, (37, 100)
    L = N + cap
    bits, dout = draw(B, L, seed=4141)
    flat = {n: bits[n].reshape(1, B * L, 24, 128) for n in "qkv"}
    cu = [0]
    for b in range(B):
        cu += [b * L + N + valid[b], (b + 1) * L]
    log(f"varlen bwd padded batch cu={cu}")
    dq, dk, dv = run_varlen_bwd(flat, dout.reshape(1, B * L, 24, 128), cu, cu)
    ref = varlen_attention_bwd(widen(flat["q"][0]), widen(flat["k"][0]), widen(flat["v"][0]),
                               widen(dout.reshape(B * L, 24, 128)), cu, cu)
    for i, (name, got) in enumerate((("dq", dq), ("dk", dk), ("dv", dv))):
        log(f"  {name} {grad_close(widen(got), ref[i], name)}")
