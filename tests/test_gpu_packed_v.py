"""GPU checks of the packed-V path of the attention forward calls.

With a workspace, hv_joint_attention_fwd / hv_attention_fwd_lse /
hv_joint_attention_varlen_fwd first rewrite V tile by tile channel-major into
it and read each P V operand with one 16-byte LDS read; without one they read
V in place with the transposing LDS read.  Both feed the same values into the
same MFMA slots, so the outputs (and log-sum-exps) must agree bit for bit.
Calls whose query blocks all fit in one round of workgroups (at most one per
CU: 256 on MI355X) read V in place even with a workspace, so the shapes here
carry enough batch entries or rows to make the call pack.

* bitwise agreement of the two paths on small shapes around the 64-key tile
  (ragged tails, one key, exact multiples of 64, batch entries with different
  valid lengths), on the log-sum-exp form with its own K/V length, and on
  packed segments with empty ones in between;
* bitwise agreement of the 4-wave variant that calls with few query blocks
  run (128-row blocks) with the 8-wave blocks of larger calls;
* the workspace holds exactly the documented packed layout (per segment,
  head and tile: 128 channel rows of 64 keys, keys swapped in bits 2 and 3
  inside each group of 16, zeros past the valid keys), then the work counter
  through which the persistent workgroups took the query blocks (it ends at
  blocks + workgroups: every workgroup's last take finds no block), and
  nothing past the bytes the call needs is written;
* one workspace reused by two calls in a row, the second smaller; poisoned
  padded rows never reach the workspace; a too-small workspace is refused.
Parity with the fp64 oracle for the packed path is covered by every other GPU
attention test, which run it by default.
"""
import numpy as np
import pytest

import hvinputs
from hvtest_util import assert_close, bits_to_torch, log, torch_to_bits, widen
from oracle import joint_attention

pytestmark = pytest.mark.gpu

TILE = 64 * 128  # elements of one (head, tile) block


def key_of_pos(p):
    p = np.asarray(p)
    return (p & ~15) | (p & 3) | (((p >> 3) & 1) << 2) | (((p >> 2) & 1) << 3)


def expected_packed(vbits, k_lens, k_offs):
    """The packed layout for segments (k_off row, k_len) of v[rows, 24, 128]."""
    blocks = []
    pos = np.arange(64)
    for k0, n in zip(k_offs, k_lens):
        nt = (n + 63) // 64
        for h in range(24):
            for t in range(nt):
                keys = 64 * t + key_of_pos(pos)
                blk = np.zeros((128, 64), np.uint16)
                ok = keys < n
                blk[:, ok] = vbits[k0 + keys[ok], h, :].T
                blocks.append(blk.reshape(-1))
    return np.concatenate(blocks) if blocks else np.zeros(0, np.uint16)


SHAPES = [
    # batch, n_video, text capacity, valid text per batch entry; every shape
    # has more than 256 query blocks of 256 rows (24 per entry and 256 rows)
    (11, 1, 0, [0] * 11),                        # one key
    (11, 40, 24, [24] * 11),                     # exactly one tile
    (11, 40, 25, [24, 25] * 5 + [0]),            # 64 keys, one padded row
    (11, 63, 2, [0, 2] * 5 + [1]),               # keys 63 and 65
    (6, 200, 57, [13, 57, 0, 1, 56, 30]),
    (6, 300, 45, [45, 3, 0, 44, 1, 2]),
    (2, 2047, 256, [255, 1]),
]


def packed_workspace(n_video, valid):
    """A workspace of exactly the packed-V size."""
    import torch

    need = sum((n_video + x + 63) // 64 for x in valid) * 24 * TILE * 2 + 256
    return torch.empty(need, dtype=torch.uint8, device="cuda")


def blocks_of(B, L):
    return 24 * B * ((L + 255) // 256)


@pytest.mark.parametrize("B,n_video,cap,valid", SHAPES, ids=lambda x: str(x))
def test_packed_and_inplace_paths_agree_bitwise(B, n_video, cap, valid):
    import torch
    import rope_joint_attention_amd as hv

    L = n_video + cap
    assert blocks_of(B, L) > 256
    bits = hvinputs.draw_qkv(B, L, seed=31 * L + B)
    q, k, v = (bits_to_torch(bits[n]) for n in ("q", "k", "v"))
    log(f"packed vs in-place B={B} N={n_video} L={L} valid={valid}")
    a = hv.hv_joint_attention_fwd(q, k, v, valid, n_video, workspace=packed_workspace(n_video, valid))
    b = hv.hv_joint_attention_fwd(q, k, v, valid, n_video, pack_v=False)
    torch.cuda.synchronize()
    assert np.array_equal(torch_to_bits(a), torch_to_bits(b))
    ref = joint_attention(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), n_video, valid)
    assert_close(widen(torch_to_bits(a)), ref, f"packed B={B} L={L}")


def test_lse_form_agrees_bitwise():
    import torch
    import rope_joint_attention_amd as hv

    bq = hvinputs.draw_qkv(2, 1400, seed=91)      # 2 x 6 x 24 = 288 query blocks
    bk = hvinputs.draw_qkv(2, 517, seed=92)
    q = bits_to_torch(bq["q"])
    k, v = bits_to_torch(bk["k"]), bits_to_torch(bk["v"])
    log("packed vs in-place: lse form, 1400 queries x 517 keys, valid 517 / 130")
    oa, la = hv.hv_attention_fwd_lse(q, k, v, [517, 130], pack_v=True)
    ob, lb = hv.hv_attention_fwd_lse(q, k, v, [517, 130], pack_v=False)
    torch.cuda.synchronize()
    assert np.array_equal(torch_to_bits(oa), torch_to_bits(ob))
    assert np.array_equal(la.cpu().numpy().view(np.uint32), lb.cpu().numpy().view(np.uint32))


def test_varlen_form_agrees_bitwise():
    import torch
    import rope_joint_attention_amd as hv

    T = 3700
    bits = hvinputs.draw_qkv(1, T, seed=93)
    q, k, v = (bits_to_torch(bits[n][0]) for n in ("q", "k", "v"))
    cq = [0, 1300, 1300, 2700, 3650]   # 6 + 6 + 4 query blocks per head: 384
    ck = [0, 2000, 2600, 3000, 3700]   # segment 1 has keys but no queries
    log(f"packed vs in-place: varlen cu_q={cq} cu_k={ck}")
    oa, la = hv.hv_joint_attention_varlen_fwd(q, k, v, cq, ck, want_lse=True, pack_v=True)
    ob, lb = hv.hv_joint_attention_varlen_fwd(q, k, v, cq, ck, want_lse=True, pack_v=False)
    torch.cuda.synchronize()
    a, b = torch_to_bits(oa), torch_to_bits(ob)
    assert np.array_equal(a[:3650], b[:3650])
    la, lb = la.cpu().numpy(), lb.cpu().numpy()
    assert np.array_equal(la[:, :3650].view(np.uint32), lb[:, :3650].view(np.uint32))


@pytest.mark.parametrize("na", [1, 333, 1100])
def test_small_call_variant_agrees_bitwise(na):
    # Calls whose 128-row query blocks all fit in one round of workgroups run a
    # 4-wave variant of the kernel (one wave per SIMD).  A segment of na rows
    # computed that way (a call on it alone: ceil(na / 128) * 24 <= 256
    # blocks) equals the same segment computed inside a call that also holds a
    # 4000-row segment (8 waves per block, packed and in place), bit for bit.
    import torch
    import rope_joint_attention_amd as hv

    T = na + 4000
    bits = hvinputs.draw_qkv(1, T, seed=900 + na)
    q, k, v = (bits_to_torch(bits[n][0]) for n in ("q", "k", "v"))
    cu = [0, na, T]
    log(f"4-wave vs 8-wave blocks: segment of {na} rows, alone and beside 4000 rows")
    big_p, lse_p = hv.hv_joint_attention_varlen_fwd(q, k, v, cu, want_lse=True, pack_v=True)
    big_i, lse_i = hv.hv_joint_attention_varlen_fwd(q, k, v, cu, want_lse=True, pack_v=False)
    one, lse_1 = hv.hv_joint_attention_varlen_fwd(q[:na].contiguous(), k[:na].contiguous(),
                                                  v[:na].contiguous(), [0, na], want_lse=True)
    torch.cuda.synchronize()
    a = torch_to_bits(one)
    for big, lse in ((big_p, lse_p), (big_i, lse_i)):
        assert np.array_equal(torch_to_bits(big)[:na], a)
        assert np.array_equal(lse[:, :na].cpu().numpy().view(np.uint32), lse_1.cpu().numpy().view(np.uint32))
    ref = joint_attention(widen(bits["q"][:, :na]), widen(bits["k"][:, :na]), widen(bits["v"][:, :na]),
                          na, [0])
    assert_close(widen(a)[None], ref, f"4-wave blocks, {na} rows")


def test_workspace_holds_the_packed_layout():
    import torch
    import rope_joint_attention_amd as hv

    B, n_video, cap = 12, 150, 40                    # 12 x 24 = 288 query blocks
    valid = [40, 7] * 6                              # 190 and 157 keys: 3 tiles each
    L = n_video + cap
    assert blocks_of(B, L) > 256
    bits = hvinputs.draw_qkv(B, L, seed=94)
    vb = bits["v"].copy()
    vb[1, n_video + 7:] = 0x7FC0                     # NaN in the padded rows of entry 1
    q, k, v = bits_to_torch(bits["q"]), bits_to_torch(bits["k"]), bits_to_torch(vb)
    need = sum((n_video + x + 63) // 64 for x in valid) * 24 * TILE * 2 + 256
    cap_bytes = hv.hv_attention_workspace_bytes(B * L, B)
    assert cap_bytes >= need
    ws = torch.full((cap_bytes // 2,), 0x1234, dtype=torch.int16, device="cuda")
    log(f"packed layout B={B} L={L} valid={valid}: need {need} bytes of {cap_bytes}")
    out = hv.hv_joint_attention_fwd(q, k, v, valid, n_video, workspace=ws)
    torch.cuda.synchronize()
    got = ws.cpu().numpy().view(np.uint16)
    want = np.concatenate([expected_packed(vb[b], [n_video + valid[b]], [0]) for b in range(B)])
    assert want.size * 2 + 256 == need
    assert np.array_equal(got[:want.size], want)
    blocks = B * 24 * ((L + 255) // 256)
    groups = min(blocks, torch.cuda.get_device_properties(0).multi_processor_count)
    counter = int(got[want.size:want.size + 2].view(np.int32)[0])
    assert counter == blocks + groups
    assert (got[want.size + 2:] == 0x1234).all()      # nothing else past the packed tiles
    o = widen(torch_to_bits(out))
    assert np.isfinite(o).all()
    ref = joint_attention(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), n_video, valid)
    assert_close(o, ref, "packed layout call")


def test_varlen_workspace_layout_skips_segments_without_queries():
    import torch
    import rope_joint_attention_amd as hv

    T = 3100
    bits = hvinputs.draw_qkv(1, T, seed=95)
    q, k, v = (bits_to_torch(bits[n][0]) for n in ("q", "k", "v"))
    cq = [0, 1500, 1500, 3000]      # 6 + 6 query blocks per head: 288
    ck = [0, 70, 200, 330]          # segment 1: 130 keys, no queries -> not packed
    ws = torch.zeros(hv.hv_attention_workspace_bytes(T, 3) // 2, dtype=torch.int16, device="cuda")
    log("varlen packed layout with a query-less segment")
    hv.hv_joint_attention_varlen_fwd(q, k, v, cq, ck, workspace=ws)
    torch.cuda.synchronize()
    got = ws.cpu().numpy().view(np.uint16)
    want = expected_packed(bits["v"][0], [70, 130], [0, 200])
    assert np.array_equal(got[:want.size], want)


def test_workspace_reused_by_consecutive_calls():
    # the second (smaller) call finds the first one's packed tiles and counter
    # in the workspace and must not depend on them: it matches the same call
    # on a fresh NaN-filled workspace bit for bit.  Both calls pack V.
    import torch
    import rope_joint_attention_amd as hv

    nbytes = hv.hv_attention_workspace_bytes(2 * 1300, 2)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for B, L, valid, seed in ((2, 1300, [100, 7], 96), (3, 900, [17, 0, 120], 97)):
        assert blocks_of(B, L) > 256
        bits = hvinputs.draw_qkv(B, L, seed=seed)
        q, k, v = (bits_to_torch(bits[n]) for n in ("q", "k", "v"))
        n_video = L - 120
        log(f"workspace reuse L={L}")
        a = hv.hv_joint_attention_fwd(q, k, v, valid, n_video, workspace=ws)
        fresh = torch.full((nbytes // 2,), float("nan"), dtype=torch.bfloat16, device="cuda")
        b = hv.hv_joint_attention_fwd(q, k, v, valid, n_video, workspace=fresh)
        torch.cuda.synchronize()
        assert np.array_equal(torch_to_bits(a), torch_to_bits(b))
        ref = joint_attention(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), n_video, valid)
        assert_close(widen(torch_to_bits(a)), ref, f"reused workspace L={L}")


def test_too_small_workspace_is_refused():
    import torch
    import rope_joint_attention_amd as hv

    bits = hvinputs.draw_qkv(1, 200, seed=98)
    q, k, v = (bits_to_torch(bits[n]) for n in ("q", "k", "v"))
    ws = torch.empty(4 * 24 * TILE * 2 - 16, dtype=torch.uint8, device="cuda")   # 4 tiles needed
    with pytest.raises(hv.HvError) as ei:
        hv.hv_joint_attention_fwd(q, k, v, [50], 150, workspace=ws)
    assert ei.value.status == hv.HV_ERR_INVALID_ARG
