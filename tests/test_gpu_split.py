"""GPU parity of the key-range split that hv_joint_attention_fwd uses for
small padded calls, through the C ABI.

A call with at most 128 query blocks (24 heads x ceil(seq_len / 256) per batch
entry) and a workspace with room for it cuts every batch entry's keys into up
to 8 parts of whole 64-key tiles, runs the (part, entry) pairs as segments of
one launch into partial outputs and log-sum-exps in the workspace, and merges
them (the exact log-sum-exp combination).  Checked: every output element
against the fp64 oracle on shapes that split into 2..8 parts (ragged tails,
batch entries with different valid lengths, all-padded text, strided views
with guard rows), agreement with the unsplit in-place path within rounding,
determinism, and that a call that cannot split (one tile, or too many blocks)
is bitwise the unsplit call.
"""
import numpy as np
import pytest

import hvinputs
from hvtest_util import assert_close, bits_to_torch, errors, log, torch_to_bits, widen
from oracle import joint_attention

pytestmark = pytest.mark.gpu


def parts_of(B, L, lk):
    """Parts the library splits a padded call into (1: no split)."""
    blocks = 24 * B * ((L + 255) // 256)
    if blocks > 128:
        return 1
    nt = [(x + 63) // 64 for x in lk]
    parts = min(8, 256 // blocks, min(nt))
    if parts <= 1:
        return 1
    per = -(-max(nt) // parts)           # tiles in the longest part
    return -(-max(nt) // per)            # as few parts as give that length


CASES = [
    # batch, n_video, text capacity, valid text per entry
    (1, 256, 256, [256]),      # the 256x256 image workload's shape: 4 parts of 2 tiles
    (1, 200, 57, [13]),        # 213 keys: 4 parts, ragged last tile
    (2, 300, 45, [45, 3]),     # different valid lengths, 2 parts
    (1, 900, 124, [100]),      # 4 query blocks: 2 parts of 8 tiles
    (1, 1000, 100, [0]),       # 5 query blocks, all text padded
    (1, 520, 0, [0]),          # 3 query blocks, 9 tiles: 3 parts of 3
    (1, 70, 60, [60]),         # one query block, 130 keys: 3 parts (1, 1, 1 tiles)
]


@pytest.mark.parametrize("B,n_video,cap,valid", CASES, ids=lambda x: str(x))
def test_split_matches_oracle(B, n_video, cap, valid):
    import torch
    import rope_joint_attention_amd as hv

    L = n_video + cap
    lk = [n_video + x for x in valid]
    parts = parts_of(B, L, lk)
    assert parts >= 2
    bits = hvinputs.draw_qkv(B, L, seed=17 * L + B)
    q, k, v = (bits_to_torch(bits[n]) for n in ("q", "k", "v"))
    log(f"split B={B} L={L} valid={valid}: {parts} parts")
    ws = torch.empty(hv.hv_attention_workspace_bytes(B * L, B), dtype=torch.uint8, device="cuda")
    a = hv.hv_joint_attention_fwd(q, k, v, valid, n_video, workspace=ws)
    a2 = hv.hv_joint_attention_fwd(q, k, v, valid, n_video, workspace=ws)
    b = hv.hv_joint_attention_fwd(q, k, v, valid, n_video, pack_v=False)
    torch.cuda.synchronize()
    a, a2, b = torch_to_bits(a), torch_to_bits(a2), torch_to_bits(b)
    assert np.array_equal(a, a2)                      # deterministic
    ref = joint_attention(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), n_video, valid)
    e = assert_close(widen(a), ref, f"split B={B} L={L}")
    log(f"  split {e}; unsplit {errors(widen(b), ref)}")
    # the partial results are rounded to bf16 before the merge: within a
    # few bf16 steps of the unsplit path, nowhere near the gates
    assert errors(widen(a), widen(b))["rel_fro"] <= 4e-3


def test_calls_that_cannot_split_are_unchanged():
    import torch
    import rope_joint_attention_amd as hv

    for B, n_video, cap, valid in ((1, 40, 24, [10]),          # one key tile
                                   (2, 63, 2, [0, 2]),          # an entry with one tile
                                   (3, 1300, 37, [37, 0, 5])):  # 144 query blocks
        L = n_video + cap
        assert parts_of(B, L, [n_video + x for x in valid]) == 1
        bits = hvinputs.draw_qkv(B, L, seed=5 * L + B)
        q, k, v = (bits_to_torch(bits[n]) for n in ("q", "k", "v"))
        log(f"no split B={B} L={L}")
        a = hv.hv_joint_attention_fwd(q, k, v, valid, n_video)
        b = hv.hv_joint_attention_fwd(q, k, v, valid, n_video, pack_v=False)
        torch.cuda.synchronize()
        assert np.array_equal(torch_to_bits(a), torch_to_bits(b))


def test_split_into_strided_output_leaves_guard_rows():
    import torch
    import rope_joint_attention_amd as hv

    B, n_video, cap, valid = 2, 300, 40, [40, 11]
    L = n_video + cap
    assert parts_of(B, L, [n_video + x for x in valid]) == 2
    bits = hvinputs.draw_qkv(B, L, seed=151)

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
    ref = joint_attention(widen(bits["q"]), widen(bits["k"]), widen(bits["v"]), n_video, valid)
    assert_close(widen(torch_to_bits(ob[:, 1:L + 1])), ref, "split, strided output")
