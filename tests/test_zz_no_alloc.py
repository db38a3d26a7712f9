"""The allocation-free backward (hv_joint_attention_bwd_noalloc) against
hv_joint_attention_bwd, through the C ABI.

Both run the same kernels; the no-alloc call keeps -D, -lse/scale and the
work counters in the library's static device scratch instead of a caller's
workspace, so the gradients must agree bit for bit.  Two calls in a row, the
second smaller: the scratch still holds the first call's values and counters
when the second starts, and the second must not depend on them.  The first
call is at the scratch's size limit (batch x seq_len = 174762 rows).
"""
import numpy as np
import pytest

import hvinputs
from hvtest_util import bits_to_torch, log, torch_to_bits, widen

pytestmark = pytest.mark.gpu


def _compare(B, L, N, valid, seed):
    import torch
    import rope_joint_attention_amd as hv

    log(f"no-alloc backward B={B} L={L} N={N} valid={valid} seed={seed}")
    bits = hvinputs.draw_qkv(B, L, seed)
    q, k, v = (bits_to_torch(bits[n]) for n in "qkv")
    g = bits_to_torch(hvinputs.draw_qkv(B, L, seed + 7919)["q"])
    del bits
    lk = [N + x for x in valid]
    out, lse = hv.hv_attention_fwd_lse(q, k, v, lk)
    ref = hv.hv_joint_attention_bwd(q, k, v, out, g, lse, list(valid), N)
    got = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    hv.hv_joint_attention_bwd_noalloc(q, k, v, out, g, lse, list(valid), N, *got)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
    # and the gradients are the gradients: every padded key gets zero
    for b_ in range(B):
        n = N + valid[b_]
        assert not widen(torch_to_bits(got[1][b_, n:])).any()
        assert not widen(torch_to_bits(got[2][b_, n:])).any()
    assert np.isfinite(widen(torch_to_bits(got[0][:, :64]))).all()


def test_noalloc_backward_matches_the_workspace_backward_twice():
    import rope_joint_attention_amd as hv

    rows = (hv.HV_NOALLOC_BWD_SCRATCH_BYTES - 256) // (2 * 24 * 4)
    _compare(1, rows, rows - 256, (200,), 701)      # the whole scratch
    _compare(2, 700, 640, (60, 13), 702)            # smaller, right after


def test_noalloc_backward_refuses_more_than_the_scratch():
    import torch
    import rope_joint_attention_amd as hv

    rows = (hv.HV_NOALLOC_BWD_SCRATCH_BYTES - 256) // (2 * 24 * 4) + 1
    q = torch.zeros((1, rows, 24, 128), dtype=torch.bfloat16, device="cuda")
    t = [torch.zeros_like(q) for _ in range(7)]
    lse = torch.zeros((1, 24, rows), dtype=torch.float32, device="cuda")
    with pytest.raises(hv.HvError) as e:
        hv.hv_joint_attention_bwd_noalloc(q, t[0], t[1], t[2], t[3], lse, [256], rows - 256,
                                          t[4], t[5], t[6])
    assert e.value.status == hv.HV_ERR_UNSUPPORTED
