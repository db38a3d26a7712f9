"""Helpers shared by the GPU parity tests (not a test module)."""
from __future__ import annotations

import math

import numpy as np

# Tolerances.  The workload definition fixes max-abs <= 2e-2 and mean-abs <= 2e-3
# against the fp64 oracle for bf16 inputs with fp32 accumulation.  Because
# attention outputs shrink like sqrt(e / L_k) for unit-normal inputs, a relative
# Frobenius gate is added; a correct bf16-output kernel sits near 2^-9 relative.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_FRO = 1e-2


def bits_to_torch(bits: np.ndarray, device="cuda"):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def torch_to_bits(t) -> np.ndarray:
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def widen(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray) -> dict:
    d = np.abs(got - ref)
    return {
        "max_abs": float(d.max()) if d.size else 0.0,
        "mean_abs": float(d.mean()) if d.size else 0.0,
        "rel_fro": float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)),
        "nonfinite": int((~np.isfinite(got)).sum()),
    }


def assert_close(got: np.ndarray, ref: np.ndarray, what: str, rel_fro: float = REL_FRO,
                 max_abs: float = MAX_ABS, mean_abs: float = MEAN_ABS) -> dict:
    e = errors(got, ref)
    msg = f"{what}: {e}"
    assert e["nonfinite"] == 0, msg
    assert e["max_abs"] <= max_abs, msg
    assert e["mean_abs"] <= mean_abs, msg
    assert e["rel_fro"] <= rel_fro, msg
    return e


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def log(msg: str) -> None:
    print(msg, flush=True)
