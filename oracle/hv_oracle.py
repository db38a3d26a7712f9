"""fp64 reference implementation (test infrastructure; see package docstring).

Citations name the HunyuanVideo notes page ("HunyuanVideo 模型结构与数学原理",
note.shouss.top, page 1 of the source set) and the summary page of the
technical report (zhao9797.github.io, "hunyuan-video"), by section.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

HEADS = 24       # notes page, section 5.1: hidden 3072 = 24 heads x 128
HEAD_DIM = 128

# Notes page section 5.5 / report summary Table 2: per-head channels split
# (d_t, d_h, d_w) = (16, 56, 56) in that order.  (axis, first channel, width)
ROPE_AXES = (("t", 0, 16), ("h", 16, 56), ("w", 72, 56))


@dataclasses.dataclass(frozen=True)
class OracleGrid:
    frames: int
    height: int
    width: int
    t_lat: int   # T'
    h_lat: int   # H' = H / 8
    w_lat: int   # W' = W / 8
    gt: int      # token grid along time   = T'
    gh: int      # token grid along height = H' / 2
    gw: int      # token grid along width  = W' / 2
    n_video: int


def token_grid(frames: int, height: int, width: int) -> OracleGrid:
    """Latent and token grid of an F x H x W clip.

    Notes page section 4: the causal VAE compresses time by 4 and space by 8,
    valid for F = 4k + 1, giving T' = floor((F - 1) / 4) + 1, H' = H / 8,
    W' = W / 8; the 1x2x2 patch embedding then gives
    N = T' * (H' / 2) * (W' / 2).  Section 8 checks that the frame size is a
    multiple of 16 and the frame count is 4k + 1 before running.
    """
    for name, val in (("frames", frames), ("height", height), ("width", width)):
        if not isinstance(val, (int, np.integer)) or val <= 0:
            raise ValueError(f"{name} must be a positive integer, got {val!r}")
    if (frames - 1) % 4 != 0:
        raise ValueError(f"frames must be 4k+1, got {frames}")
    if height % 16 != 0 or width % 16 != 0:
        raise ValueError(f"height and width must be multiples of 16, got {height}x{width}")
    t_lat = (frames - 1) // 4 + 1
    h_lat = height // 8
    w_lat = width // 8
    gt, gh, gw = t_lat, h_lat // 2, w_lat // 2
    return OracleGrid(frames, height, width, t_lat, h_lat, w_lat, gt, gh, gw, gt * gh * gw)


def rope_frequencies(theta: float):
    """Per-axis rotation frequencies theta^(-2j/d_a), j < d_a/2.

    Section 5.5 writes R_3D as the direct sum R_t + R_h + R_w of one-dimensional
    rotary embeddings (RoFormer); each axis block uses the RoFormer frequencies
    over its own width d_a.  Returned as {axis: float64 array}.
    """
    out = {}
    for axis, _off, d in ROPE_AXES:
        j = np.arange(d // 2, dtype=np.float64)
        out[axis] = np.power(np.float64(theta), -2.0 * j / d)
    return out


def video_coordinates(grid: OracleGrid) -> np.ndarray:
    """Integer (t, h, w) patch coordinates of every video token, shape [N, 3].

    The patchified latent is flattened t-major then row-major (a meshgrid
    over the T' x H'/2 x W'/2 grid), coordinates start at 0 with unit step.
    """
    t, h, w = np.meshgrid(np.arange(grid.gt), np.arange(grid.gh), np.arange(grid.gw),
                          indexing="ij")
    return np.stack([t.reshape(-1), h.reshape(-1), w.reshape(-1)], axis=1).astype(np.int64)


def apply_rope3d(x: np.ndarray, token_index: np.ndarray, grid: OracleGrid,
                 theta: float) -> np.ndarray:
    """Rotate the rows of ``x`` that are video tokens; return a float64 copy.

    ``x``: float64 [..., R, HEADS, HEAD_DIM]; ``token_index``: [R] sequence
    position of each row.  Rows with position >= N (text) are returned
    unchanged.  For a video token with coordinates (t, h, w), every head's
    channel pair (o_a + 2j, o_a + 2j + 1) of axis block a is rotated by the
    angle pos_a * theta^(-2j/d_a):
        x0' = x0 cos(phi) - x1 sin(phi),  x1' = x0 sin(phi) + x1 cos(phi).
    Only Q and K are passed through here; V is never rotated (section 5.5:
    RoPE is applied to the visual Q, K only).
    """
    x = np.array(x, dtype=np.float64, copy=True)
    token_index = np.asarray(token_index, dtype=np.int64)
    assert x.shape[-3] == token_index.shape[0] and x.shape[-1] == HEAD_DIM
    coords = video_coordinates(grid)
    freqs = rope_frequencies(theta)
    video_rows = np.nonzero(token_index < grid.n_video)[0]
    chunk = 4096
    for s in range(0, video_rows.size, chunk):
        rows = video_rows[s:s + chunk]
        pos = coords[token_index[rows]]                  # [r, 3]
        for a, (axis, off, d) in enumerate(ROPE_AXES):
            phi = pos[:, a:a + 1].astype(np.float64) * freqs[axis][None, :]   # [r, d/2]
            c = np.cos(phi)[:, None, :]                  # broadcast over heads
            sn = np.sin(phi)[:, None, :]
            sel = x[..., rows, :, off:off + d]
            x0 = sel[..., 0::2].copy()
            x1 = sel[..., 1::2].copy()
            sel[..., 0::2] = x0 * c - x1 * sn
            sel[..., 1::2] = x0 * sn + x1 * c
            x[..., rows, :, off:off + d] = sel
    return x


def rms_norm_heads(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Per-head RMSNorm, float64 (notes page section 5.4).

    Each head vector x (the last axis, d = 128 channels) becomes
        gamma * x / sqrt(mean_j(x_j^2) + eps).
    ``gamma`` broadcasts against ``x`` (a [128] vector, or one per row).
    """
    x = np.asarray(x, dtype=np.float64)
    mean_sq = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64) * (x / np.sqrt(mean_sq + eps))


def qk_norm_rope3d(x: np.ndarray, token_index: np.ndarray, grid: OracleGrid, theta: float,
                   gamma_video: np.ndarray, gamma_text: Optional[np.ndarray],
                   eps: float) -> np.ndarray:
    """QK-norm prologue of the attention: per-head RMSNorm, then 3D RoPE.

    Section 5.4 normalises every head of Q and K with an RMSNorm; section 5.2
    keeps separate parameters for the video and text streams in the
    double-stream blocks, so video rows use ``gamma_video`` and text rows
    ``gamma_text`` (the same vector when it is None, as in the single-stream
    blocks of section 5.3).  Section 5.5 then rotates the video rows.
    ``x``: float64 [..., R, HEADS, HEAD_DIM] holding the rows listed in
    ``token_index``.  Returns a float64 array of the same shape.
    """
    token_index = np.asarray(token_index, dtype=np.int64)
    gv = np.asarray(gamma_video, dtype=np.float64)
    gt = gv if gamma_text is None else np.asarray(gamma_text, dtype=np.float64)
    is_video = token_index < grid.n_video
    g = np.where(is_video[:, None], gv[None, :], gt[None, :])[:, None, :]   # [R, 1, D]
    y = rms_norm_heads(x, g, eps)
    return apply_rope3d(y, token_index, grid, theta)


def joint_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_video: int,
                    valid: Sequence[int], scale: Optional[float] = None,
                    rows: Optional[np.ndarray] = None,
                    heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """Exact joint softmax attention, float64.

    Section 5.2: Q = [Q_v; Q_t], K = [K_v; K_t], V = [V_v; V_t] along the
    sequence (video first) and Attn = softmax(Q K^T / sqrt(128)) V per head.
    Text keys at positions >= n_video + valid[b] are padding and are excluded
    from the softmax.  Every query row (padded text rows included) attends to
    the same valid keys.

    ``q``: float64 [B, Rq, H, D] holding the query rows listed in ``rows``
    (all L rows when ``rows`` is None); ``k``, ``v``: float64 [B, L, H, D].
    Returns float64 [B, Rq, H', D] for the heads listed in ``heads``.
    """
    B, L, H, D = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if heads is None:
        heads = range(H)
    heads = list(heads)
    Rq = q.shape[1]
    out = np.zeros((B, Rq, len(heads), D), dtype=np.float64)
    for b in range(B):
        lk = n_video + int(valid[b])
        if lk <= 0:
            raise ValueError("no valid keys")
        for hi, h in enumerate(heads):
            kb = np.ascontiguousarray(k[b, :lk, h, :])
            vb = np.ascontiguousarray(v[b, :lk, h, :])
            for s in range(0, Rq, 256):
                qb = q[b, s:s + 256, h, :]
                scores = (qb @ kb.T) * scale
                m = scores.max(axis=1, keepdims=True)
                p = np.exp(scores - m)
                z = p.sum(axis=1, keepdims=True)
                out[b, s:s + 256, hi, :] = (p @ vb) / z
    return out


def attention_lse(q: np.ndarray, k: np.ndarray, v: np.ndarray, k_len: Sequence[int],
                  scale: Optional[float] = None,
                  heads: Optional[Sequence[int]] = None):
    """Exact softmax attention of every query row against the first k_len[b]
    keys of batch entry b, with the log-sum-exp of its logits, float64.

    ``q``: [B, Rq, H, D]; ``k``, ``v``: [B, Lk, H, D] (Rq and Lk independent,
    as when a rank of a sequence-parallel ring holds its own query rows and
    receives another rank's K/V block: notes page section 9.2).  Returns
    (out [B, Rq, H', D], lse [B, H', Rq]) with
        lse_i = log sum_j exp(scale * q_i . k_j),   out_i = sum_j exp(s_ij - lse_i) v_j.
    """
    B, Lk, H, D = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    heads = list(range(H)) if heads is None else list(heads)
    Rq = q.shape[1]
    out = np.zeros((B, Rq, len(heads), D), dtype=np.float64)
    lse = np.zeros((B, len(heads), Rq), dtype=np.float64)
    for b in range(B):
        n = int(k_len[b])
        if n <= 0 or n > Lk:
            raise ValueError("k_len out of range")
        for hi, h in enumerate(heads):
            kb = np.ascontiguousarray(k[b, :n, h, :])
            vb = np.ascontiguousarray(v[b, :n, h, :])
            for s0 in range(0, Rq, 256):
                scores = (q[b, s0:s0 + 256, h, :] @ kb.T) * scale
                m = scores.max(axis=1, keepdims=True)
                p = np.exp(scores - m)
                z = p.sum(axis=1, keepdims=True)
                out[b, s0:s0 + 256, hi, :] = (p @ vb) / z
                lse[b, hi, s0:s0 + 256] = (m + np.log(z))[:, 0]
    return out, lse


def merge_partials(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray]):
    """Combine attention results over disjoint key sets into the result over
    their union, float64 (the Ring Attention half of USP, notes page section
    9.2: each rank keeps its query rows and sees the K/V blocks one at a time).

    For parts i with outputs O_i [B, R, H, D] and log-sum-exps lse_i [B, H, R]:
        lse = log sum_i exp(lse_i),   O = sum_i exp(lse_i - lse) O_i.
    This is the softmax over the union written per part, since part i's
    unnormalised numerator is exp(lse_i) O_i.  Returns (O, lse).
    """
    lses = np.stack([np.asarray(x, dtype=np.float64) for x in lses])        # [P, B, H, R]
    outs = np.stack([np.asarray(x, dtype=np.float64) for x in outs])        # [P, B, R, H, D]
    top = lses.max(axis=0)
    w = np.exp(lses - top)                                                  # [P, B, H, R]
    total = w.sum(axis=0)
    lse = top + np.log(total)
    wt = np.transpose(w / total, (0, 1, 3, 2))[..., None]                   # [P, B, R, H, 1]
    return (wt * outs).sum(axis=0), lse


def varlen_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     cu_q: Sequence[int], cu_k: Sequence[int],
                     scale: Optional[float] = None,
                     heads: Optional[Sequence[int]] = None):
    """Exact attention over packed segments, float64 (the variable-length form
    of FlashAttention that the model calls, notes page section 9.1).

    ``q``, ``k``, ``v``: [T, H, D] packed rows.  Segment s owns query rows
    [cu_q[s], cu_q[s+1]) and key rows [cu_k[s], cu_k[s+1]); its queries attend
    to its keys only.  Returns (out [T, H', D], lse [H', T]); rows outside
    every segment are left zero in both.
    """
    T, H, D = q.shape
    heads = list(range(H)) if heads is None else list(heads)
    out = np.zeros((T, len(heads), D), dtype=np.float64)
    lse = np.zeros((len(heads), T), dtype=np.float64)
    for s in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        if q1 == q0:
            continue
        o, l = attention_lse(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], [k1 - k0],
                             scale=scale, heads=heads)
        out[q0:q1] = o[0]
        lse[:, q0:q1] = l[0]
    return out, lse


def joint_attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                        n_video: int, valid: Sequence[int], scale: Optional[float] = None,
                        heads: Optional[Sequence[int]] = None):
    """Gradients of the joint attention of ``joint_attention``, float64.

    With O = softmax(scale * Q K^T) V over the valid keys of each batch entry
    (the attention the report summary page names as the training bottleneck,
    "FusedAttention" in its Infra section) and an upstream gradient dO, the
    chain rule through the softmax gives, per (batch, head):
        P  = softmax(scale * Q K^T),       dV = P^T dO,
        dP = dO V^T,                        dS = P * (dP - rowsum(P * dP)),
        dQ = scale * dS K,                  dK = scale * dS^T Q.
    Padded keys take no part, so their dK, dV are zero.  All query rows
    (padded text rows included) contribute, as in the forward.
    ``q``, ``k``, ``v``, ``dout``: [B, L, H, D].  Returns (dq, dk, dv), each
    [B, L, H', D] for the heads listed in ``heads``.
    """
    B, L, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    heads = list(range(H)) if heads is None else list(heads)
    dq = np.zeros((B, L, len(heads), D), dtype=np.float64)
    dk = np.zeros_like(dq)
    dv = np.zeros_like(dq)
    for b in range(B):
        lk = n_video + int(valid[b])
        if lk <= 0:
            raise ValueError("no valid keys")
        for hi, h in enumerate(heads):
            qb, kb, vb, gb = (np.ascontiguousarray(t[b, :, h, :]) for t in (q, k, v, dout))
            kb, vb = kb[:lk], vb[:lk]
            s = (qb @ kb.T) * scale
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = gb @ vb.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[b, :, hi, :] = scale * (ds @ kb)
            dk[b, :lk, hi, :] = scale * (ds.T @ qb)
            dv[b, :lk, hi, :] = p.T @ gb
    return dq, dk, dv


def joint_attention_bwd_dq_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                                n_video: int, valid: Sequence[int],
                                scale: Optional[float] = None,
                                heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """dQ of ``joint_attention_bwd`` for a subset of query rows.

    A query row's gradient needs only its own softmax row: P_i over the valid
    keys, dP_i = dO_i V^T and dS_i = P_i * (dP_i - sum_j P_ij dP_ij), then
    dQ_i = scale * dS_i K.  ``q`` and ``dout`` hold the selected rows
    ([B, R, H, D]); ``k``, ``v`` all rows.  Returns [B, R, H', D].
    """
    B, L, H, D = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    heads = list(range(H)) if heads is None else list(heads)
    R = q.shape[1]
    dq = np.zeros((B, R, len(heads), D), dtype=np.float64)
    for b in range(B):
        lk = n_video + int(valid[b])
        for hi, h in enumerate(heads):
            kb = np.ascontiguousarray(k[b, :lk, h, :])
            vb = np.ascontiguousarray(v[b, :lk, h, :])
            for s0 in range(0, R, 256):
                qb = q[b, s0:s0 + 256, h, :]
                gb = dout[b, s0:s0 + 256, h, :]
                sc = (qb @ kb.T) * scale
                p = np.exp(sc - sc.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                dp = gb @ vb.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, s0:s0 + 256, hi, :] = scale * (ds @ kb)
    return dq


def joint_attention_bwd_by_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                                n_video: int, valid: Sequence[int], scale: Optional[float] = None,
                                heads: Optional[Sequence[int]] = None,
                                batches: Optional[Sequence[int]] = None, chunk: int = 256,
                                workers: int = 1):
    """Gradients of ``joint_attention_bwd`` for long sequences, float64.

    The same chain rule, written per query row i of one (batch, head) over the
    valid keys j (the report summary page's training-side attention, the
    forward of notes page section 5.2):
        P_i   = softmax_j(scale * q_i . k_j)     (the whole row, every valid key)
        dP_ij = dO_i . v_j,   D_i = sum_j P_ij dP_ij,   dS_ij = P_ij (dP_ij - D_i)
        dQ_i  = scale * sum_j dS_ij k_j
    while each key gradient is a sum over the query rows,
        dV_j = sum_i P_ij dO_i,   dK_j = scale * sum_i dS_ij q_i,
    so it is added up over consecutive chunks of ``chunk`` query rows, in
    chunk order.  Only a chunk x L_k block of P is held per chunk, which is
    what lets the oracle check every gradient element at the longest
    workloads (one L x L_k matrix there is over 100 GB).  Padded keys get
    zero dK, dV.  ``workers`` > 1 computes that many chunks at once on
    threads (single-threaded BLAS each); the sums are still taken in chunk
    order (only the rounding inside the library's matrix products can
    differ with the thread count).

    ``q``, ``k``, ``v``, ``dout``: [B, L, H, D].  Returns (dq, dk, dv), each
    [len(batches), L, len(heads), D] for the listed batch entries and heads.
    """
    from concurrent.futures import ThreadPoolExecutor

    B, L, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    heads = list(range(H)) if heads is None else list(heads)
    batches = list(range(B)) if batches is None else list(batches)
    shape = (len(batches), L, len(heads), D)
    dq, dk, dv = (np.zeros(shape, dtype=np.float64) for _ in range(3))

    def one_chunk(qc, gc, kb, vb):
        p = (qc @ kb.T) * scale
        p -= p.max(axis=1, keepdims=True)
        np.exp(p, out=p)
        p /= p.sum(axis=1, keepdims=True)
        dp = gc @ vb.T
        d = (p * dp).sum(axis=1, keepdims=True)
        dp -= d
        dp *= p                                   # dS of the chunk
        return scale * (dp @ kb), scale * (dp.T @ qc), p.T @ gc

    limit = None
    if workers > 1:
        try:
            from threadpoolctl import threadpool_limits
            limit = threadpool_limits(1)
        except ImportError:  # pragma: no cover
            limit = None
    try:
        with ThreadPoolExecutor(max_workers=max(1, workers)) as pool:
            for bi, b in enumerate(batches):
                lk = n_video + int(valid[b])
                if lk <= 0:
                    raise ValueError("no valid keys")
                for hi, h in enumerate(heads):
                    kb = np.ascontiguousarray(k[b, :lk, h, :], dtype=np.float64)
                    vb = np.ascontiguousarray(v[b, :lk, h, :], dtype=np.float64)
                    starts = list(range(0, L, chunk))
                    pending = []
                    for i in range(len(starts) + 1):
                        if i < len(starts):
                            s0 = starts[i]
                            qc = np.ascontiguousarray(q[b, s0:s0 + chunk, h, :], dtype=np.float64)
                            gc = np.ascontiguousarray(dout[b, s0:s0 + chunk, h, :], dtype=np.float64)
                            pending.append((s0, pool.submit(one_chunk, qc, gc, kb, vb)))
                        # consume in chunk order, keeping at most 2 x workers in flight
                        while pending and (len(pending) > 2 * max(1, workers) or i == len(starts)):
                            s0, fut = pending.pop(0)
                            dqc, dkc, dvc = fut.result()
                            dq[bi, s0:s0 + chunk, hi, :] = dqc
                            dk[bi, :lk, hi, :] += dkc
                            dv[bi, :lk, hi, :] += dvc
    finally:
        if limit is not None:
            limit.unregister() if hasattr(limit, "unregister") else limit.restore_original_limits()
    return dq, dk, dv


def varlen_attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
                         cu_q: Sequence[int], cu_k: Sequence[int],
                         scale: Optional[float] = None,
                         heads: Optional[Sequence[int]] = None):
    """Gradients of ``varlen_attention`` (packed segments), float64.

    Each segment is an independent attention (its queries, its keys), so its
    gradients are those of ``joint_attention_bwd`` on that segment alone with
    every key valid.  ``q``, ``k``, ``v``, ``dout``: [T, H, D].  Returns
    (dq, dk, dv), each [T, H', D]; rows outside every segment stay zero.
    """
    T, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    heads = list(range(H)) if heads is None else list(heads)
    dq = np.zeros((T, len(heads), D), dtype=np.float64)
    dk = np.zeros_like(dq)
    dv = np.zeros_like(dq)
    for s in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        if q1 == q0:
            continue
        for hi, h in enumerate(heads):
            qb, gb = q[q0:q1, h, :], dout[q0:q1, h, :]
            kb, vb = k[k0:k1, h, :], v[k0:k1, h, :]
            sc = (qb @ kb.T) * scale
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = gb @ vb.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[q0:q1, hi, :] = scale * (ds @ kb)
            dk[k0:k1, hi, :] = scale * (ds.T @ qb)
            dv[k0:k1, hi, :] = p.T @ gb
    return dq, dk, dv


def hot_path(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
             frames: int, height: int, width: int, valid: Sequence[int],
             theta: float, rows: Optional[np.ndarray] = None,
             heads: Optional[Sequence[int]] = None, scale: Optional[float] = None):
    """Token grid -> 3D RoPE on video Q, K -> joint attention, all float64.

    ``*_bits``: bfloat16 bit patterns [B, L, H, D] (uint16), widened exactly.
    Returns (grid, out) with out float64 [B, len(rows), H', D].
    """
    from hvinputs import bf16_bits_to_f64  # storage decoding only

    grid = token_grid(frames, height, width)
    B, L = k_bits.shape[:2]
    if rows is None:
        rows = np.arange(L)
    rows = np.asarray(rows, dtype=np.int64)
    qf = apply_rope3d(bf16_bits_to_f64(q_bits[:, rows]), rows, grid, theta)
    kf = apply_rope3d(bf16_bits_to_f64(k_bits), np.arange(L), grid, theta)
    vf = bf16_bits_to_f64(v_bits)
    out = joint_attention(qf, kf, vf, grid.n_video, valid, scale=scale, heads=heads)
    return grid, out
