"""Seeded synthetic inputs for the joint video+text attention path.

This module is shared by the fp64 oracle (``oracle/``), the tests, ``bench.py``
and ``__graft_entry__.smoke``.  It holds *no* arithmetic of the method itself:
no token-grid formula, no rotary embedding, no attention.  It only knows

* the five workload definitions (clip size, batch, text lengths, seed, theta);
* how to draw Q, K, V ~ N(0, 1) from NumPy's PCG64 and round them to bfloat16
  bit patterns (round-to-nearest-even, done with integer arithmetic);
* how to widen bfloat16 bit patterns back to float32 / float64 (exact);
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

    Inputs here are finite normal draws, so NaN handling is not needed; it is
    still kept sane (a NaN stays a NaN) for poisoned-input tests.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # process in slabs to bound temporary memory for multi-GB tensors
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    slab = 1 << 24
    for s in range(0, flat_u.size, slab):
        w = flat_u[s:s + slab].astype(np.uint32)
        nan = (w & 0x7FFFFFFF) > 0x7F800000
        lsb = (w >> 16) & 1
        r = (w + np.uint32(0x7FFF) + lsb) >> 16
        r = np.where(nan, (w >> 16) | 0x40, r)
        flat_o[s:s + slab] = r.astype(np.uint16)
    return out


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

def draw_qkv(batch: int, seq_len: int, seed: int,
             heads: int = HEADS, head_dim: int = HEAD_DIM,
             q_scale: float = 1.0) -> Dict[str, np.ndarray]:
    """Q, K, V as bfloat16 bit patterns, shape [batch, seq_len, heads, head_dim].

    Draw order is q, k, v from one PCG64 stream seeded with ``seed``; each is a
    float32 standard normal (optionally scaled, for the peaky-softmax stress
    case) rounded to bfloat16.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (batch, seq_len, heads, head_dim)
    out = {}
    for name in ("q", "k", "v"):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        if name == "q" and q_scale != 1.0:
            x *= np.float32(q_scale)
        out[name] = f32_to_bf16_bits(x)
        del x
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
