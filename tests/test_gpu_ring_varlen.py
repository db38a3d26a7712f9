"""GPU parity of the sequence-parallel and packed attention entry points
(hv_attention_fwd_lse, hv_attention_merge, hv_joint_attention_varlen_fwd)
against the fp64 oracle, through the C ABI.

Outputs use the attention gates (max-abs 2e-2, mean-abs 2e-3, relative
Frobenius 1e-2, no NaN/Inf).  The log-sum-exp is compared per element within
4e-3: the kernel sums bf16-rounded weights (relative error at most 2^-9, whose
log is below 2e-3) and forms the logits in fp32.
"""
import numpy as np
import pytest

import hvinputs
from hvtest_util import assert_close, bits_to_torch, log, torch_to_bits, widen
from oracle import (attention_lse, merge_partials, token_grid,
                    varlen_attention)

pytestmark = pytest.mark.gpu
LSE_TOL = 4e-3


def lse_close(got, ref, what):
    d = np.abs(np.asarray(got, np.float64) - ref)
    assert np.isfinite(got).all(), what
    assert d.max() <= LSE_TOL, f"{what}: lse max err {d.max()}"
    return float(d.max())


@pytest.mark.parametrize("B,Lq,Lk,valid,fused_kv,scale", [
    (1, 1, 1, None, False, None),
    (1, 40, 200, None, False, None),
    (2, 300, 129, (129, 64), True, None),     # K/V as views of a fused buffer, ragged keys
    (3, 257, 513, (1, 500, 513), False, 0.05),
    (1, 512, 64, None, True, 0.3),            # peaky
])
def test_attention_lse_small(B, Lq, Lk, valid, fused_kv, scale):
    import torch
    import rope_joint_attention_amd as hv

    qb = hvinputs.draw_qkv(B, Lq, seed=Lq * 7 + Lk)["q"]
    kvb = hvinputs.draw_qkv(B, Lk, seed=Lk * 11 + Lq)
    log(f"lse small B={B} Lq={Lq} Lk={Lk} valid={valid} fused={fused_kv} scale={scale}")
    q = bits_to_torch(qb)
    if fused_kv:
        fused = torch.zeros((B, Lk, 3, 24, 128), dtype=torch.bfloat16, device="cuda")
        fused[:, :, 1] = bits_to_torch(kvb["k"])
        fused[:, :, 2] = bits_to_torch(kvb["v"])
        k, v = fused[:, :, 1], fused[:, :, 2]
    else:
        k, v = bits_to_torch(kvb["k"]), bits_to_torch(kvb["v"])
    out, lse = hv.hv_attention_fwd_lse(q, k, v, valid, softmax_scale=scale)
    torch.cuda.synchronize()
    kl = [Lk] * B if valid is None else list(valid)
    ref, lref = attention_lse(widen(qb), widen(kvb["k"]), widen(kvb["v"]), kl, scale=scale)
    assert_close(widen(torch_to_bits(out)), ref, "attention_lse out")
    lse_close(lse.cpu().numpy(), lref, "attention_lse")


def ring(q, k, v, bounds, valid_total):
    """K/V blocks [bounds[i], bounds[i+1]) as a ring would deliver them; blocks
    with no valid key are skipped, as a rank would skip them."""
    import rope_joint_attention_amd as hv

    outs, lses = [], []
    for a, b in zip(bounds, bounds[1:]):
        n = min(b, valid_total) - a
        if n <= 0:
            continue
        o, l = hv.hv_attention_fwd_lse(q, k[:, a:b], v[:, a:b], [n] * q.shape[0])
        outs.append(o)
        lses.append(l)
    return hv.hv_attention_merge(outs, lses)


@pytest.mark.parametrize("Lq,Lk,parts", [(300, 300, 2), (513, 777, 5), (64, 1000, 16), (100, 70, 1)])
def test_ring_merge_small(Lq, Lk, parts):
    import torch

    bits = hvinputs.draw_qkv(1, max(Lq, Lk), seed=Lq + Lk + parts)
    qb, kb, vb = bits["q"][:, :Lq], bits["k"][:, :Lk], bits["v"][:, :Lk]
    q, k, v = bits_to_torch(qb), bits_to_torch(kb), bits_to_torch(vb)
    bounds = sorted(set([0, Lk] + [int(x) for x in np.linspace(0, Lk, parts + 1)[1:-1]]))
    log(f"ring small Lq={Lq} Lk={Lk} blocks={bounds}")
    out, lse = ring(q, k, v, bounds, Lk)
    torch.cuda.synchronize()
    ref, lref = attention_lse(widen(qb), widen(kb), widen(vb), [Lk])
    assert_close(widen(torch_to_bits(out)), ref, "ring merge out")
    lse_close(lse.cpu().numpy(), lref, "ring merge")
    # the oracle's own merge of the oracle's block results agrees too
    po = [attention_lse(widen(qb), widen(kb[:, a:b]), widen(vb[:, a:b]), [b - a]) for a, b in
          zip(bounds, bounds[1:])]
    mo, ml = merge_partials([p[0] for p in po], [p[1] for p in po])
    assert np.allclose(mo, ref, atol=1e-12) and np.allclose(ml, lref, atol=1e-12)


def test_merge_single_part_is_identity_bitwise():
    import torch
    import rope_joint_attention_amd as hv

    bits = hvinputs.draw_qkv(2, 333, seed=9)
    q, k, v = (bits_to_torch(bits[n]) for n in "qkv")
    o, l = hv.hv_attention_fwd_lse(q, k, v)
    m, ml = hv.hv_attention_merge([o], [l])
    torch.cuda.synchronize()
    assert torch.equal(m, o) and torch.equal(ml, l)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,parts", [("video_544x960x129", 4), ("video_720x1280x129", 8),
                                        ("video_720x1280x33_b2", 3)])
def test_ring_merge_workloads(name, parts):
    # The whole hot path with the attention split into `parts` K/V blocks:
    # rope, then one hv_attention_fwd_lse per block and a merge, against the
    # oracle's fp64 rope + joint attention on sampled rows.
    import torch
    import rope_joint_attention_amd as hv
    from oracle import hot_path

    wl = hvinputs.WORKLOADS[name]
    g = token_grid(wl.frames, wl.height, wl.width)
    L = g.n_video + wl.text_capacity
    log(f"ring workload {name} B={wl.batch} L={L} parts={parts}")
    bits = hvinputs.draw_qkv(wl.batch, L, wl.seed)
    q, k, v = (bits_to_torch(bits[n]) for n in "qkv")
    hv.hv_rope3d_apply(q, k, hv.hv_token_grid(wl.frames, wl.height, wl.width), wl.theta)
    bounds = [int(x) for x in np.linspace(0, L, parts + 1)]
    # per batch entry the valid key count differs: run the ring per entry
    outs = []
    for b in range(wl.batch):
        o, _ = ring(q[b:b + 1], k[b:b + 1], v[b:b + 1], bounds, g.n_video + wl.valid[b])
        outs.append(o)
    out = torch.cat(outs, 0)
    torch.cuda.synchronize()
    ob = torch_to_bits(out)
    rows = hvinputs.sample_rows(L, g.n_video, g.gh * g.gw, wl.seed, n_random=48, edge=8)
    _, ref = hot_path(bits["q"], bits["k"], bits["v"], wl.frames, wl.height, wl.width, wl.valid,
                      wl.theta, rows=rows)
    e = assert_close(widen(ob[:, rows]), ref, f"{name} ring x{parts}")
    log(f"  {e}")


def clip_pack(clips, seed):
    """Pack clips (F, H, W, text_valid) as [video | valid text] segments."""
    lens, grids = [], []
    for F, H, W, t in clips:
        g = token_grid(F, H, W)
        grids.append(g)
        lens.append(g.n_video + t)
    T = sum(lens)
    bits = hvinputs.draw_qkv(1, T, seed)
    cu = [0] + list(np.cumsum(lens))
    return bits, grids, cu, T


def test_varlen_packed_clips():
    import torch
    import rope_joint_attention_amd as hv

    clips = [(1, 64, 64, 13), (5, 48, 80, 0), (1, 256, 256, 200), (9, 32, 48, 77)]
    bits, grids, cu, T = clip_pack(clips, seed=21)
    log(f"varlen clips T={T} cu={cu}")
    q, k, v = (bits_to_torch(bits[n])[0] for n in "qkv")
    out, lse = hv.hv_joint_attention_varlen_fwd(q, k, v, cu, want_lse=True)
    torch.cuda.synchronize()
    ref, lref = varlen_attention(widen(bits["q"][0]), widen(bits["k"][0]), widen(bits["v"][0]), cu, cu)
    assert_close(widen(torch_to_bits(out)), ref, "varlen clips out")
    lse_close(lse.cpu().numpy(), lref, "varlen clips")
    # each clip equals the joint attention call on that clip alone
    for s, ((F, H, W, t), g) in enumerate(zip(clips, grids)):
        a, b = cu[s], cu[s + 1]
        sl = slice(a, b)
        one = hv.hv_joint_attention_fwd(q[None, sl].contiguous(), k[None, sl].contiguous(),
                                        v[None, sl].contiguous(), [t], g.n_video)
        torch.cuda.synchronize()
        assert torch.equal(one[0], out[sl]), f"clip {s} differs from its own joint call"


def test_varlen_rows_outside_segments_untouched_and_cross_segments():
    import torch
    import rope_joint_attention_amd as hv

    T = 700
    bits = hvinputs.draw_qkv(1, T, seed=31)
    q, k, v = (bits_to_torch(bits[n])[0] for n in "qkv")
    cq = [0, 100, 100, 400, 650]       # an empty segment; rows 650.. belong to none
    ck = [0, 50, 60, 600, 700]         # keys of segments 2 and 3 start elsewhere
    out = torch.full_like(q, float("nan"))
    lse = torch.full((24, T), float("nan"), dtype=torch.float32, device="cuda")
    hv.hv_joint_attention_varlen_fwd(q, k, v, cq, ck, out=out, lse=lse)
    torch.cuda.synchronize()
    ref, lref = varlen_attention(widen(bits["q"][0]), widen(bits["k"][0]), widen(bits["v"][0]), cq, ck)
    ob = widen(torch_to_bits(out))
    assert np.isnan(ob[650:]).all() and torch.isnan(lse[:, 650:]).all()
    assert_close(ob[:650], ref[:650], "varlen cross segments")
    lse_close(lse[:, :650].cpu().numpy(), lref[:, :650], "varlen cross segments")


@pytest.mark.timeout(600)
def test_varlen_padded_batch_matches_oracle():
    # The padded two-entry workload flattened into [valid | padded tail]
    # segments: valid rows are the joint attention, each tail attends to itself.
    import torch
    import rope_joint_attention_amd as hv

    wl = hvinputs.WORKLOADS["video_720x1280x33_b2"]
    g = token_grid(wl.frames, wl.height, wl.width)
    L = g.n_video + wl.text_capacity
    bits = hvinputs.draw_qkv(wl.batch, L, wl.seed)
    flat = {n: bits[n].reshape(wl.batch * L, 24, 128) for n in "qkv"}
    cu = [0]
    for b in range(wl.batch):
        cu += [b * L + g.n_video + wl.valid[b], (b + 1) * L]
    log(f"varlen padded batch cu={cu}")
    q, k, v = (bits_to_torch(flat[n]) for n in "qkv")
    out, lse = hv.hv_joint_attention_varlen_fwd(q, k, v, cu, want_lse=True)
    torch.cuda.synchronize()
    ob = torch_to_bits(out)
    rows = hvinputs.sample_rows(L, g.n_video, g.gh * g.gw, wl.seed, n_random=48, edge=8)
    for b in range(wl.batch):
        n = g.n_video + wl.valid[b]
        r = rows + b * L
        seg_rows = r[rows < n]
        ref, lref = attention_lse(widen(flat["q"][None, seg_rows]), widen(flat["k"][None, b * L:b * L + n]),
                                  widen(flat["v"][None, b * L:b * L + n]), [n])
        assert_close(widen(ob[seg_rows]), ref[0], f"entry {b} valid rows")
        lse_close(lse[:, seg_rows].cpu().numpy(), lref[0], f"entry {b} valid rows")
        if n < L:
            tail = np.arange(b * L + n, (b + 1) * L)
            ref, _ = attention_lse(widen(flat["q"][None, tail]), widen(flat["k"][None, tail]),
                                   widen(flat["v"][None, tail]), [tail.size])
            assert_close(widen(ob[tail]), ref[0], f"entry {b} padded tail")


def test_varlen_maximum_segment_count():
    # HV_MAX_SEGMENTS packed segments of ragged lengths, some empty
    import torch
    import rope_joint_attention_amd as hv

    r = np.random.default_rng(64)
    lens = [int(x) for x in r.integers(0, 40, size=hv.HV_MAX_SEGMENTS)]
    lens[5] = 0
    lens[-1] = 1
    cu = [0] + list(np.cumsum(lens))
    T = cu[-1]
    bits = hvinputs.draw_qkv(1, T, seed=6464)
    log(f"varlen {len(lens)} segments T={T}")
    q, k, v = (bits_to_torch(bits[n])[0] for n in "qkv")
    out, lse = hv.hv_joint_attention_varlen_fwd(q, k, v, cu, want_lse=True)
    torch.cuda.synchronize()
    ref, lref = varlen_attention(widen(bits["q"][0]), widen(bits["k"][0]), widen(bits["v"][0]), cu, cu)
    assert_close(widen(torch_to_bits(out)), ref, "varlen 64 segments")
    lse_close(lse.cpu().numpy(), lref, "varlen 64 segments")


def test_merge_maximum_part_count():
    import torch
    import rope_joint_attention_amd as hv

    Lq, Lk, P = 130, 1600, hv.HV_MAX_MERGE_PARTS
    bits = hvinputs.draw_qkv(2, Lk, seed=1616)
    qb, kb, vb = bits["q"][:, :Lq], bits["k"], bits["v"]
    q, k, v = bits_to_torch(qb), bits_to_torch(kb), bits_to_torch(vb)
    bounds = [int(x) for x in np.linspace(0, Lk, P + 1)]
    outs, lses = [], []
    for a, b in zip(bounds, bounds[1:]):
        o, l = hv.hv_attention_fwd_lse(q, k[:, a:b], v[:, a:b])
        outs.append(o)
        lses.append(l)
    out, lse = hv.hv_attention_merge(outs, lses)
    torch.cuda.synchronize()
    ref, lref = attention_lse(widen(qb), widen(kb), widen(vb), [Lk, Lk])
    assert_close(widen(torch_to_bits(out)), ref, "merge of 16 parts")
    lse_close(lse.cpu().numpy(), lref, "merge of 16 parts")
