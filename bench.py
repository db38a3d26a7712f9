#!/usr/bin/env python3
"""Benchmark of the joint video+text attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one pass of the whole hot path over one synthetic batch:
hv_token_grid -> hv_rope3d_apply (video Q/K, in place) -> hv_joint_attention_fwd
(with its packed-V workspace: the call packs V, then runs the attention; the
attention time reported covers both kernels, so the roofline figure slightly
understates the attention kernel alone).
Inputs are generated on the host and copied to HBM before timing.  RoPE
works in place, so every step gets a fresh batch: warmup + steps copies of
the unrotated Q and K are staged in HBM beforehand (33.6 GB at
720x1280x129 with the defaults; the part has 288 GB), and step i rotates copy
i and runs the attention on it.  V, the output and the workspace are shared.
The JSON records the SHA-256 of the input bytes and the host's core count.

Printed: ONE JSON line (stdout) with the whole-step throughput in attention
TFLOP/s (algorithmic FLOPs 4*heads*head_dim*sum_b L*Lk_b over the step time),
per-kernel times from HIP events on the launch stream, the attention
kernel's MFMA roofline fraction, and the fp64 oracle timed on a bounded
sample of the same workload on the host cores.  The QK-norm + RoPE prologue
(hv_qk_norm_rope3d_apply, all rows of q and k) is timed separately on the
same resident tensors and reported beside the step (qknorm_rope_*).  The
`extras` object times one rank's share of an 8-way ring attention (partial
attention per K/V block plus the log-sum-exp merge), a packed
variable-length call and the attention backward (--no-extras skips them).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "joint-attn TFLOP/s, ms/call and % MFMA peak at 720×1280×129 (L=119056)"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
HEADS, HEAD_DIM = 24, 128


def progress(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attn_flops(batch: int, seq_len: int, lk) -> float:
    return 4.0 * HEADS * HEAD_DIM * sum(float(seq_len) * x for x in lk)


def kernel_source_hash() -> str:
    """Hash of the attention kernel's code with comments and blank lines removed,
    so that a comment edit does not invalidate recorded counters."""
    p = os.path.join(ROOT, "rope_joint_attention_amd", "csrc", "attn_fwd.hip")
    text = re.sub(r"/\*.*?\*/", "", open(p).read(), flags=re.S)
    code = [ln.split("//", 1)[0].rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in code if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary,
    only if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not b or h.group(1) != kernel_source_hash():
        return None
    return float(b.group(1))


def cpu_baseline(bits, wl, n_video, seq_len, rows_n: int):
    """The fp64 oracle (unchanged) on a bounded sample: rows_n query rows of every
    head and batch entry, against all keys, including its RoPE of all of K."""
    import numpy as np

    from oracle import hot_path

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    nproc = host_cores()
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    rows = np.sort(rng.choice(seq_len, size=rows_n, replace=False))
    t0 = time.perf_counter()
    hot_path(bits["q"], bits["k"], bits["v"], wl.frames, wl.height, wl.width, wl.valid, wl.theta,
             rows=rows)
    dt = time.perf_counter() - t0
    lk = [n_video + v for v in wl.valid]
    flops = 4.0 * HEADS * HEAD_DIM * rows_n * sum(lk)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "host_cores": nproc,
        "kind": "oracle",
        "sample": (f"{rows_n} random query rows x {HEADS} heads x batch {wl.batch} against all "
                   f"{max(lk)} keys of {wl.name}, incl. fp64 RoPE of all K; {dt:.1f} s; "
                   f"'cores' = the BLAS threads its matrix products ran on (its elementwise "
                   f"steps run on one), of the {nproc} host cores this process may use"),
        "seconds": dt,
    }


def host_cores() -> int:
    """Host cores this process may run on (nproc)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def timed(torch, stream, fn, reps: int) -> float:
    """Average ms of fn() over reps calls, HIP events on the launch stream."""
    fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        fn()
    ev[1].record(stream)
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


def graph_timed(torch, fn, calls: int, reps: int) -> float:
    """Average ms of one fn() call with `calls` calls captured in one HIP graph
    and the graph replayed `reps` times: the GPU's time per call without the
    host's per-call launch work (which sets the eager time of small calls)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        g.replay()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / (reps * calls)
    del g
    return ms


def extra_rows(hv, hvinputs, torch, np, q, k, v, wl, grid, L, stream, reps: int) -> dict:
    """Measurements of the sequence-parallel and packed attention forms on the
    resident tensors (not part of the timed step).

    ring8_rank: one rank's share of an 8-way ring at this size: L/8 query
      rows against the 8 K/V blocks of L/8 keys (8 hv_attention_fwd_lse calls)
      plus the hv_attention_merge of the 8 partial results.
    merge8: that merge alone, against HBM (reads 8 partial outputs and
      log-sum-exps, writes one of each).
    varlen_pack: the batch of two 720x1280x33 clips with 37 and 256 valid text
      tokens packed as [valid | padded tail] segments of one sequence (the
      padded tails attend to themselves), one hv_joint_attention_varlen_fwd.
    workloads: attention and RoPE of each of the five workloads (device-side
      random inputs of the workload's shape, timing only), each call with its
      workspace allocated beforehand: `attn_ms` eager calls back to back,
      `attn_ms_graph` calls replayed from a HIP graph (the GPU time per call
      without the host's launch work, which dominates the eager time of the
      smallest workload); the TFLOP/s and % of peak use the graph time.
    backward: hv_joint_attention_bwd at this size.  `tflops` counts the usual
      five matrix products of an attention backward (2.5x the forward's
      FLOPs); the kernels execute seven (S and dP are formed twice, once for
      dK/dV and once for dQ), reported as `tflops_executed`.
    """
    out = {}
    P = 8
    Lr = L // P
    bounds = [i * Lr for i in range(P)] + [L]
    valid_total = grid.n_video + wl.valid[0]
    qr = q[:1, :Lr]
    parts = []
    for a, b in zip(bounds, bounds[1:]):
        n = min(b, valid_total) - a
        if n > 0:
            parts.append((a, b, n))
    po = [torch.empty_like(qr) for _ in parts]
    pl = [torch.empty((1, HEADS, Lr), dtype=torch.float32, device=q.device) for _ in parts]
    mo = torch.empty_like(qr)
    ml = torch.empty((1, HEADS, Lr), dtype=torch.float32, device=q.device)

    def partials():
        for (a, b, n), o, l in zip(parts, po, pl):
            hv.hv_attention_fwd_lse(qr, k[:1, a:b], v[:1, a:b], [n], out=o, lse=l)

    def merge():
        hv.hv_attention_merge(po, pl, out=mo, lse_out=ml)

    ms_part = timed(torch, stream, partials, reps)
    ms_merge = timed(torch, stream, merge, reps)
    fl = 4.0 * HEADS * HEAD_DIM * Lr * sum(n for _, _, n in parts)
    mbytes = (len(parts) + 1) * (Lr * HEADS * HEAD_DIM * 2 + Lr * HEADS * 4)
    out["ring8_rank"] = {"q_rows": Lr, "kv_blocks": len(parts), "ms": round(ms_part + ms_merge, 4),
                         "attn_ms": round(ms_part, 4),
                         "tflops": round(fl / ((ms_part + ms_merge) / 1e3) / 1e12, 2),
                         "attn_tflops": round(fl / (ms_part / 1e3) / 1e12, 2)}
    out["merge8"] = {"ms": round(ms_merge, 4), "bytes": mbytes,
                     "GBps": round(mbytes / (ms_merge / 1e3) / 1e9, 1),
                     "pct_hbm_peak": round(100.0 * mbytes / (ms_merge / 1e3) / 1e9 / PEAK_HBM_GBPS, 2)}
    del po, pl, mo, ml

    wb = hvinputs.WORKLOADS["video_720x1280x33_b2"]
    gb = hv.hv_token_grid(wb.frames, wb.height, wb.width)
    Lb = gb.n_video + wb.text_capacity
    T = wb.batch * Lb
    if T <= q.shape[1]:
        qp, kp, vp = (t[0, :T] for t in (q, k, v))
        cu = [0]
        seg_pairs = []
        for b in range(wb.batch):
            n = gb.n_video + wb.valid[b]
            cu += [b * Lb + n, (b + 1) * Lb]
            seg_pairs += [n * n, (Lb - n) ** 2]
        op = torch.empty_like(qp)
        ms_v = timed(torch, stream, lambda: hv.hv_joint_attention_varlen_fwd(qp, kp, vp, cu, out=op), reps)
        flv = 4.0 * HEADS * HEAD_DIM * sum(seg_pairs)
        out["varlen_pack"] = {"workload": wb.name, "segments": len(cu) - 1, "rows": T,
                              "ms": round(ms_v, 4), "tflops": round(flv / (ms_v / 1e3) / 1e12, 2)}
        del op

    # every workload's attention and RoPE time (device-side random bf16 inputs
    # of the workload's shape; timing only)
    wlt = {}
    for name, w in hvinputs.WORKLOADS.items():
        gw = hv.hv_token_grid(w.frames, w.height, w.width)
        Lw = gw.n_video + w.text_capacity
        gen = torch.Generator(device=q.device).manual_seed(w.seed)
        qw, kw, vw = (torch.randn((w.batch, Lw, HEADS, HEAD_DIM), device=q.device, generator=gen)
                      .to(torch.bfloat16) for _ in range(3))
        ow = torch.empty_like(qw)
        wsw = torch.empty(hv.hv_attention_workspace_bytes(w.batch * Lw, w.batch), dtype=torch.uint8,
                          device=q.device)

        def call():
            hv.hv_joint_attention_fwd(qw, kw, vw, list(w.valid), gw.n_video, out=ow, workspace=wsw)

        ms_a = timed(torch, stream, call, reps)
        small = w.batch * Lw <= 16384
        ms_g = graph_timed(torch, call, 50 if small else 1, 4 if small else 2)
        ms_r = timed(torch, stream, lambda: hv.hv_rope3d_apply(qw, kw, gw, w.theta), reps)
        lkw = [gw.n_video + x for x in w.valid]
        flw = 4.0 * HEADS * HEAD_DIM * Lw * sum(lkw)
        rbytes = 4.0 * w.batch * gw.n_video * HEADS * HEAD_DIM * 2
        wlt[name] = {"seq_len": Lw, "attn_ms": round(ms_a, 4), "attn_ms_graph": round(ms_g, 4),
                     "attn_tflops": round(flw / (ms_g / 1e3) / 1e12, 2),
                     "pct_mfma_peak": round(100.0 * flw / (ms_g / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                     "rope_ms": round(ms_r, 4),
                     "rope_GBps": round(rbytes / (ms_r / 1e3) / 1e9, 1)}
        del qw, kw, vw, ow, wsw
    out["workloads"] = wlt

    # backward of the headline attention: forward with log-sum-exp once, then
    # the gradients for an upstream gradient (v's values stand in for dO)
    lk = [grid.n_video + x for x in wl.valid]
    o, lse = hv.hv_attention_fwd_lse(q, k, v, lk)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    delta = torch.empty(2 * lse.numel() + hv.BWD_COUNTER_FLOATS, dtype=torch.float32, device=q.device)
    ms_b = timed(torch, stream, lambda: hv.hv_joint_attention_bwd(
        q, k, v, o, v, lse, list(wl.valid), grid.n_video, dq=dq, dk=dk, dv=dv, delta=delta),
        max(2, reps // 2))
    fwd_fl = 4.0 * HEADS * HEAD_DIM * L * sum(lk)
    out["backward"] = {"ms": round(ms_b, 4),
                       "tflops": round(2.5 * fwd_fl / (ms_b / 1e3) / 1e12, 2),
                       "flops_counted": 2.5 * fwd_fl,
                       "tflops_executed": round(3.5 * fwd_fl / (ms_b / 1e3) / 1e12, 2)}
    del o, lse, dq, dk, dv, delta
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the ring-attention and packed-segment measurements")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the hot path is built and timed on a single "
              "MI355X (no sharding or collectives in this library); run with --gpus 1.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import hvinputs
    import rope_joint_attention_amd as hv

    hv.load_library()  # fails loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    name = args.workload or hvinputs.HEADLINE
    wl = hvinputs.WORKLOADS[name]
    grid = hv.hv_token_grid(wl.frames, wl.height, wl.width)
    L = grid.n_video + wl.text_capacity
    lk = [grid.n_video + v for v in wl.valid]
    progress(f"workload {name}: B={wl.batch} L={L} N={grid.n_video} valid={list(wl.valid)}")

    t0 = time.perf_counter()
    bits = hvinputs.draw_qkv(wl.batch, L, wl.seed)
    progress(f"inputs drawn in {time.perf_counter() - t0:.1f} s")

    def to_dev(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    inputs_sha = hvinputs.sha256_of((bits["q"], bits["k"], bits["v"]))
    q, k, v = to_dev(bits["q"]), to_dev(bits["k"]), to_dev(bits["v"])
    # one unrotated copy of q and k per step (RoPE rotates in place)
    n_copies = args.warmup + args.steps
    qs = [q] + [q.clone() for _ in range(n_copies - 1)]
    ks = [k] + [k.clone() for _ in range(n_copies - 1)]
    progress(f"{n_copies} copies of q and k staged in HBM")
    out = torch.empty_like(q)
    # the forward's packed-V workspace, allocated once like the tensors
    ws = torch.empty(hv.hv_attention_workspace_bytes(wl.batch * L, wl.batch), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def step(i, ev=None):
        g = hv.hv_token_grid(wl.frames, wl.height, wl.width)
        if ev is not None:
            ev[0].record(stream)
        hv.hv_rope3d_apply(qs[i], ks[i], g, wl.theta)
        if ev is not None:
            ev[1].record(stream)
        hv.hv_joint_attention_fwd(qs[i], ks[i], v, list(wl.valid), g.n_video, out=out, workspace=ws)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    progress(f"warmup {args.warmup} done")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rope_ms = [e[0].elapsed_time(e[1]) for e in events]
    attn_ms = [e[1].elapsed_time(e[2]) for e in events]
    progress(f"timed {args.steps} steps in {wall:.2f} s")
    # every timed call saw the same rotated inputs
    for i in range(1, args.steps):
        assert torch.equal(qs[args.warmup], qs[args.warmup + i])
    q, k = qs[-1], ks[-1]
    del qs[:-1], ks[:-1]
    torch.cuda.empty_cache()

    # The QK-norm + RoPE prologue (an alternative to the RoPE step that also
    # normalises every row): timed on its own, on the same resident q and k.
    gam = {n: to_dev(b) for n, b in hvinputs.draw_gamma(wl.seed).items()}
    g0 = hv.hv_token_grid(wl.frames, wl.height, wl.width)

    def prologue():
        hv.hv_qk_norm_rope3d_apply(q, k, g0, wl.theta, gam["q_video"], gam["k_video"],
                                   gam["q_text"], gam["k_text"], 1e-6)

    for _ in range(2):
        prologue()
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        pev[i][0].record(stream)
        prologue()
        pev[i][1].record(stream)
    torch.cuda.synchronize()
    qkn_ms = [e[0].elapsed_time(e[1]) for e in pev]
    progress(f"timed {args.steps} QK-norm + RoPE prologue calls")

    # context for the HBM-bound kernels: a plain device-to-device copy of
    # 1 GiB (torch's copy kernel), read + write bytes over its event time
    csrc = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(csrc)
    copy_ms = timed(torch, stream, lambda: cdst.copy_(csrc), 5)
    copy_gbps = 2.0 * csrc.numel() * 4 / (copy_ms / 1000.0) / 1e9
    del csrc, cdst

    if args.copy_ref_mib > 0:
        n = args.copy_ref_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        progress(f"reference copy of {args.copy_ref_mib} MiB done (x3)")

    flops = attn_flops(wl.batch, L, lk)
    ms_step = wall * 1000.0 / args.steps
    attn_avg = float(np.mean(attn_ms))
    rope_avg = float(np.mean(rope_ms))
    achieved = flops / (attn_avg / 1000.0) / 1e12
    rope_bytes = 4.0 * wl.batch * grid.n_video * HEADS * HEAD_DIM * 2
    rope_gbps = rope_bytes / (rope_avg / 1000.0) / 1e9
    traffic = recorded_traffic(name)
    qkn_avg = float(np.mean(qkn_ms))
    qkn_bytes = 4.0 * wl.batch * L * HEADS * HEAD_DIM * 2
    qkn_gbps = qkn_bytes / (qkn_avg / 1000.0) / 1e9

    result = {
        "metric": METRIC,
        "value": round(flops / (ms_step / 1000.0) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "inputs_sha256": inputs_sha,
        "host_cores": host_cores(),
        "config": {"workload": name, "batch": wl.batch, "seq_len": L, "n_video": grid.n_video,
                   "text_valid": list(wl.valid), "heads": HEADS, "head_dim": HEAD_DIM,
                   "theta": wl.theta, "frames_hw": [wl.frames, wl.height, wl.width]},
        "attn_ms_per_call": round(attn_avg, 4),
        "attn_ms_min": round(float(np.min(attn_ms)), 4),
        "attn_tflops": round(achieved, 2),
        "pct_mfma_peak": round(100.0 * achieved / PEAK_BF16_TFLOPS, 2),
        "rope_ms_per_call": round(rope_avg, 4),
        "rope_GBps": round(rope_gbps, 1),
        "rope_pct_hbm_peak": round(100.0 * rope_gbps / PEAK_HBM_GBPS, 2),
        "attn_flops_per_call": flops,
        "qknorm_rope_ms_per_call": round(qkn_avg, 4),
        "qknorm_rope_GBps": round(qkn_gbps, 1),
        "qknorm_rope_pct_hbm_peak": round(100.0 * qkn_gbps / PEAK_HBM_GBPS, 2),
        "hbm_copy_GBps": round(copy_gbps, 1),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    if not args.no_extras:
        result["extras"] = extra_rows(hv, hvinputs, torch, np, q, k, v, wl, grid, L, stream,
                                      max(3, args.steps // 4))
    del q, k, v, out
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        progress("timing the fp64 oracle on a bounded sample (host cores)")
        cb = cpu_baseline(bits, wl, grid.n_video, L, args.cpu_rows)
        cb.pop("seconds", None)
        cb["value"] = round(cb["value"], 6)
        result["cpu_baseline"] = cb
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
