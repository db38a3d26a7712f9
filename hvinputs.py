"""Seeded synthetic inputs for the joint video+text attention path.

This module is shared by the fp64 oracle (``oracle/``), the tests, ``bench.py``
and ``__graft_entry__.smoke``.  It holds *no* arithmetic of the method itself:
no token-grid formula, no rotary embedding, no attention.  It only knows

* the five workload definitions (clip size, batch, text lengths, seed, theta);
* how to draw Q, K, V ~ N(0, 1) from NumPy's PCG64 and round them to bfloat16
  bit patterns (round-to-nearest-even, done with integer arithmetic);
* how to widen bfloat16 bit patterns back to float32 / float64 (exact);
* how to draw synthetic RMSNorm weights (near one) for the QK-norm prologue;
* a deterministic query-row sampler used where the full fp64 oracle would be
  too slow.

Sequence lengths are *not* computed here: callers pass ``seq_len`` (= video
tokens + text capacity), which they obtain from their own token-grid function.

The workloads follow the HunyuanVideo notes page ("HunyuanVideo 模型结构与数学原理"):
544x960x17 and 720x1280x129 clips appear in its section 4, the 256-token text
budget in section 3.1 and the 24 x 128 head geometry in section 5.1.  Q and K
come out of a per-head RMSNorm in that model (section 5.4), so unit-variance
normal draws are the stand-in for real activations.
"""
from __future__ import annotations

import dataclasses
import os
from typing import Dict, Iterable, List, Sequence

import numpy as np

HEADS = 24
HEAD_DIM = 128
TEXT_CAPACITY = 256  # prompt tokens kept by the text encoder branch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark / parity configuration.

    ``valid`` holds the number of valid (non-padding) text tokens per batch
    element; text tokens beyond it are key padding.
    """

    name: str
    frames: int
    height: int
    width: int
    batch: int
    valid: tuple
    seed: int
    theta: float = 10000.0
    text_capacity: int = TEXT_CAPACITY
    description: str = ""


WORKLOADS: Dict[str, Workload] = {
    "image_256x256": Workload(
        "image_256x256", 1, 256, 256, 1, (256,), 1001,
        description="single image (F=1) at 256x256, all 256 text tokens valid"),
    "video_544x960x17": Workload(
        "video_544x960x17", 17, 544, 960, 1, (256,), 1002,
        description="544x960, 17 frames, all text valid"),
    "video_720x1280x33_b2": Workload(
        "video_720x1280x33_b2", 33, 720, 1280, 2, (37, 256), 1003,
        description="batch 2 at 720x1280x33, text valid lengths 37 and 256"),
    "video_544x960x129": Workload(
        "video_544x960x129", 129, 544, 960, 1, (180,), 1004,
        description="544x960, 129 frames, 180 of 256 text tokens valid"),
    "video_720x1280x129": Workload(
        "video_720x1280x129", 129, 720, 1280, 1, (256,), 1005,
        description="720x1280, 129 frames, all text valid (largest single clip)"),
}

# Order used by tests and reports (smallest first).
WORKLOAD_ORDER: List[str] = list(WORKLOADS)
HEADLINE = "video_720x1280x129"


# --------------------------------------------------------------------------
# bfloat16 bit handling (storage format only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns (round to nearest, ties to even).

    NaN inputs stay NaN (quieted); infinities stay infinite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = x.view(np.uint32)
    r = ((w + ((w >> 16) & 1) + np.uint32(0x7FFF)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((w[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64 (exact)."""
    return bf16_bits_to_f32(bits).astype(np.float64)


# --------------------------------------------------------------------------
# seeded draws
# --------------------------------------------------------------------------

CHUNK = 1 << 22  # elements per independent random stream


def _draw_chunk(seed: int, tensor: int, chunk: int, n: int, scale: float) -> np.ndarray:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(tensor, chunk))
    x = np.random.Generator(np.random.PCG64(ss)).standard_normal(size=n, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return f32_to_bf16_bits(x)


def draw_qkv(batch: int, seq_len: int, seed: int,
             heads: int = HEADS, head_dim: int = HEAD_DIM,
             q_scale: float = 1.0, workers: int = 0) -> Dict[str, np.ndarray]:
    """Q, K, V as bfloat16 bit patterns, shape [batch, seq_len, heads, head_dim].

    Each tensor (q = 0, k = 1, v = 2) is flattened row-major and cut into
    chunks of CHUNK elements; chunk i of tensor t holds float32 standard
    normals from PCG64(SeedSequence(seed, spawn_key=(t, i))), rounded to
    bfloat16.  Q is optionally scaled first (peaky-softmax stress case).
    Chunks are independent, so they are drawn on a thread pool; the values
    do not depend on the number of workers.
    """
    from concurrent.futures import ThreadPoolExecutor

    shape = (batch, seq_len, heads, head_dim)
    total = int(np.prod(shape))
    if workers <= 0:
        workers = max(1, min(16, os.cpu_count() or 1))
    out = {}
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for t, name in enumerate(("q", "k", "v")):
            flat = np.empty(total, dtype=np.uint16)
            scale = q_scale if name == "q" else 1.0
            futs = []
            for i, s in enumerate(range(0, total, CHUNK)):
                n = min(CHUNK, total - s)
                futs.append((s, n, pool.submit(_draw_chunk, seed, t, i, n, scale)))
            for s, n, f in futs:
                flat[s:s + n] = f.result()
            out[name] = flat.reshape(shape)
    return out


def draw_gamma(seed: int, head_dim: int = HEAD_DIM, spread: float = 0.25) -> Dict[str, np.ndarray]:
    """Synthetic RMSNorm weights as bfloat16 bit patterns, one [head_dim]
    vector each for video Q, video K, text Q and text K.

    Values are 1 + spread * N(0, 1) (float32 from
    PCG64(SeedSequence(seed, spawn_key=(3 + i,))) for vector i), rounded to
    bfloat16, standing in for trained weights that stay near one.
    """
    out = {}
    for i, name in enumerate(("q_video", "k_video", "q_text", "k_text")):
        ss = np.random.SeedSequence(entropy=seed, spawn_key=(3 + i,))
        x = np.random.Generator(np.random.PCG64(ss)).standard_normal(size=head_dim, dtype=np.float32)
        out[name] = f32_to_bf16_bits(np.float32(1.0) + np.float32(spread) * x)
    return out


def sample_rows(seq_len: int, n_video: int, frame_tokens: int, seed: int,
                n_random: int = 256, edge: int = 64) -> np.ndarray:
    """Deterministic query-row subset for spot checks at large sizes.

    Holds every text row (valid and padded), the first and last ``edge`` video
    rows, the rows either side of every frame boundary (``frame_tokens`` video
    tokens per frame, supplied by the caller) and ``n_random`` seeded rows.
    """
    rows = set(range(n_video, seq_len))
    rows.update(range(0, min(edge, n_video)))
    rows.update(range(max(0, n_video - edge), n_video))
    if frame_tokens > 0:
        for start in range(frame_tokens, n_video, frame_tokens):
            rows.update((start - 1, start))
    rng = np.random.Generator(np.random.PCG64(seed ^ 0x5EED))
    if n_video > 0:
        rows.update(int(r) for r in rng.integers(0, n_video, size=n_random))
    return np.array(sorted(r for r in rows if 0 <= r < seq_len), dtype=np.int64)


def sha256_of(arrays: Iterable[np.ndarray]) -> str:
    import hashlib
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).view(np.uint8).reshape(-1).data)
    return h.hexdigest()
