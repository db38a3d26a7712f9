"""GPU check that the attention calls can be captured in a HIP graph
(torch.cuda.CUDAGraph) and replayed.

The captured sequence is hv_joint_attention_fwd with a packed-V workspace,
the same call on a small batch (one round of query blocks, so it reads V in
place with one workgroup per block), hv_attention_fwd_lse with the first
workspace and hv_joint_attention_bwd with its delta workspace.  Both workspaces hold work counters that the persistent
workgroups draw blocks from; the calls reset them with a kernel of their own
(no memset node is recorded), so every replay must redo the whole work.  Each
replay runs on new inputs copied into the captured buffers, with eager calls
and synchronisations in between, and must reproduce the eager results bit for
bit (a replay that found a counter spent would leave stale outputs behind).
"""
import numpy as np
import pytest

import hvinputs
from hvtest_util import bits_to_torch, log, torch_to_bits

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_calls():
    import torch
    import rope_joint_attention_amd as hv

    B, L, N, valid = 2, 1400, 1300, [60, 13]   # 288 query blocks: V is packed
    lk = [N + x for x in valid]
    shape = (B, L, hv.HV_HEADS, hv.HV_HEAD_DIM)
    q, k, v, g = (torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(4))
    out_j, out_l = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((B, hv.HV_HEADS, L), dtype=torch.float32, device="cuda")
    ws = torch.empty(hv.hv_attention_workspace_bytes(B * L, B), dtype=torch.uint8, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    delta = torch.empty(2 * B * hv.HV_HEADS * L + hv.BWD_COUNTER_FLOATS, dtype=torch.float32, device="cuda")
    # a small call (48 query blocks, 8 key tiles): V read in place
    Ls, Ns, valid_s = 512, 256, [200]
    qs, ks, vs = (torch.empty((1, Ls, hv.HV_HEADS, hv.HV_HEAD_DIM), dtype=torch.bfloat16, device="cuda")
                  for _ in range(3))
    out_s = torch.empty_like(qs)
    ws_s = torch.empty(hv.hv_attention_workspace_bytes(Ls, 1), dtype=torch.uint8, device="cuda")

    def fill(seed):
        bits = hvinputs.draw_qkv(B, L, seed)
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            t.copy_(bits_to_torch(bits[n]))
        g.copy_(bits_to_torch(hvinputs.draw_qkv(B, L, seed + 7919)["q"]))
        small = hvinputs.draw_qkv(1, Ls, seed + 101)
        for t, n in ((qs, "q"), (ks, "k"), (vs, "v")):
            t.copy_(bits_to_torch(small[n]))

    def calls():
        hv.hv_joint_attention_fwd(q, k, v, valid, N, out=out_j, workspace=ws)
        hv.hv_joint_attention_fwd(qs, ks, vs, valid_s, Ns, out=out_s, workspace=ws_s)
        hv.hv_attention_fwd_lse(q, k, v, lk, out=out_l, lse=lse, workspace=ws)
        hv.hv_joint_attention_bwd(q, k, v, out_l, g, lse, valid, N, dq=dq, dk=dk, dv=dv, delta=delta)

    fill(80)
    side = torch.cuda.Stream()  # warm-up off the capture stream, as torch asks
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    for seed in (81, 82, 83):
        fill(seed)
        torch.cuda.synchronize()
        log(f"graph replay on inputs of seed {seed}")
        graph.replay()
        torch.cuda.synchronize()
        got = [torch_to_bits(t) for t in (out_j, out_s, out_l, dq, dk, dv)]
        got_lse = lse.cpu().numpy().view(np.uint32).copy()
        # the same calls eagerly, with fresh outputs and workspaces
        e_j = hv.hv_joint_attention_fwd(q, k, v, valid, N)
        e_s = hv.hv_joint_attention_fwd(qs, ks, vs, valid_s, Ns)
        e_l, e_lse = hv.hv_attention_fwd_lse(q, k, v, lk)
        e_g = hv.hv_joint_attention_bwd(q, k, v, e_l, g, e_lse, valid, N)
        torch.cuda.synchronize()
        want = [torch_to_bits(t) for t in (e_j, e_s, e_l, *e_g)]
        for name, a, b in zip(("out", "out (small call)", "out (lse form)", "dq", "dk", "dv"), got, want):
            assert np.array_equal(a, b), f"replay {seed}: {name} differs from the eager call"
        assert np.array_equal(got_lse, e_lse.cpu().numpy().view(np.uint32)), f"replay {seed}: lse"
