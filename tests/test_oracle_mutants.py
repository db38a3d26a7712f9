"""Mutation check of the oracle's pins.

Each mutant below is a plausible mistake in the fp64 oracle (a dropped term, a
wrong sign, index, offset or operand).  For every one, a copy of ``oracle/``
with that single edit is put beside copies of the pin tests
(tests/test_oracle_*.py and tests/golden/), and the pins are run against it in
a separate process: at least one pin must fail.  The unmutated copy must pass,
so a failure is the mutant's doing.  The edits are textual and each must
match exactly once, so a mutant that no longer applies is reported rather
than silently passing.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = "oracle/hv_oracle.py"

# (name, old text, new text), applied to oracle/hv_oracle.py
MUTANTS = [
    # token grid (notes page section 4)
    ("latent frames off by one", "t_lat = (frames - 1) // 4 + 1", "t_lat = (frames - 1) // 4"),
    ("spatial stride 16 for the latent", "h_lat = height // 8", "h_lat = height // 16"),
    # 3D RoPE (section 5.5)
    ("rotation sign", "sel[..., 0::2] = x0 * c - x1 * sn", "sel[..., 0::2] = x0 * c + x1 * sn"),
    ("frequency exponent", "np.power(np.float64(theta), -2.0 * j / d)",
     "np.power(np.float64(theta), -1.0 * j / d)"),
    ("frequency base width shared", "out[axis] = np.power(np.float64(theta), -2.0 * j / d)",
     "out[axis] = np.power(np.float64(theta), -2.0 * j / 128)"),
    ("h and w channel blocks swapped", 'ROPE_AXES = (("t", 0, 16), ("h", 16, 56), ("w", 72, 56))',
     'ROPE_AXES = (("t", 0, 16), ("h", 72, 56), ("w", 16, 56))'),
    ("axis offset", 'ROPE_AXES = (("t", 0, 16), ("h", 16, 56), ("w", 72, 56))',
     'ROPE_AXES = (("t", 0, 16), ("h", 16, 56), ("w", 70, 56))'),
    ("coordinate order", "np.stack([t.reshape(-1), h.reshape(-1), w.reshape(-1)], axis=1)",
     "np.stack([t.reshape(-1), w.reshape(-1), h.reshape(-1)], axis=1)"),
    ("half-split pairing", "x0 = sel[..., 0::2].copy()\n            x1 = sel[..., 1::2].copy()\n"
     "            sel[..., 0::2] = x0 * c - x1 * sn\n            sel[..., 1::2] = x0 * sn + x1 * c",
     "x0 = sel[..., :d // 2].copy()\n            x1 = sel[..., d // 2:].copy()\n"
     "            sel[..., :d // 2] = x0 * c - x1 * sn\n            sel[..., d // 2:] = x0 * sn + x1 * c"),
    ("text rows rotated too", "video_rows = np.nonzero(token_index < grid.n_video)[0]",
     "video_rows = np.nonzero(token_index <= grid.n_video)[0]"),
    # RMSNorm (section 5.4) and stream weights (section 5.2)
    ("epsilon outside the root", "(x / np.sqrt(mean_sq + eps))", "(x / (np.sqrt(mean_sq) + eps))"),
    ("sum of squares instead of mean", "mean_sq = np.mean(x * x, axis=-1, keepdims=True)",
     "mean_sq = np.sum(x * x, axis=-1, keepdims=True)"),
    ("stream weights swapped", "np.where(is_video[:, None], gv[None, :], gt[None, :])",
     "np.where(is_video[:, None], gt[None, :], gv[None, :])"),
    ("RoPE before the norm", "y = rms_norm_heads(x, g, eps)\n    return apply_rope3d(y, token_index, grid, theta)",
     "y = apply_rope3d(x, token_index, grid, theta)\n    return rms_norm_heads(y, g, eps)"),
    # joint attention (section 5.2)
    ("scale 1/d", "    if scale is None:\n        scale = 1.0 / math.sqrt(D)\n    if heads is None:",
     "    if scale is None:\n        scale = 1.0 / D\n    if heads is None:"),
    ("one padded key let in", "        lk = n_video + int(valid[b])\n        if lk <= 0:\n            raise ValueError(\"no valid keys\")\n        for hi, h in enumerate(heads):\n            kb = np.ascontiguousarray(k[b, :lk, h, :])\n            vb = np.ascontiguousarray(v[b, :lk, h, :])\n            for s in range(",
     "        lk = n_video + int(valid[b]) + 1\n        if lk <= 0:\n            raise ValueError(\"no valid keys\")\n        for hi, h in enumerate(heads):\n            kb = np.ascontiguousarray(k[b, :lk, h, :])\n            vb = np.ascontiguousarray(v[b, :lk, h, :])\n            for s in range("),
    ("softmax not normalised", "out[b, s:s + 256, hi, :] = (p @ vb) / z", "out[b, s:s + 256, hi, :] = (p @ vb)"),
    ("values of the wrong head", "vb = np.ascontiguousarray(v[b, :lk, h, :])\n            for s in range(0, Rq, 256):",
     "vb = np.ascontiguousarray(v[b, :lk, (h + 1) % H, :])\n            for s in range(0, Rq, 256):"),
    # log-sum-exp and merge (section 9.2)
    ("log-sum-exp without the maximum", "lse[b, hi, s0:s0 + 256] = (m + np.log(z))[:, 0]",
     "lse[b, hi, s0:s0 + 256] = np.log(z)[:, 0]"),
    ("merge weights not normalised", "wt = np.transpose(w / total, (0, 1, 3, 2))[..., None]",
     "wt = np.transpose(w, (0, 1, 3, 2))[..., None]"),
    ("merged lse linear", "lse = top + np.log(total)", "lse = top + total"),
    # packed segments (section 9.1)
    ("segment keys offset by the query rows", "o, l = attention_lse(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1], [k1 - k0],",
     "o, l = attention_lse(q[None, q0:q1], k[None, q0:q1], v[None, q0:q1], [q1 - q0],"),
    # gradients
    ("backward drops D", "ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))\n            dq[b, :, hi, :]",
     "ds = p * dp\n            dq[b, :, hi, :]"),
    ("dK from the wrong operand", "dk[b, :lk, hi, :] = scale * (ds.T @ qb)", "dk[b, :lk, hi, :] = scale * (ds.T @ gb)"),
    ("dV transposed product", "dv[b, :lk, hi, :] = p.T @ gb", "dv[b, :lk, hi, :] = p.T @ gb[::-1]"),
    ("dQ rows drop the scale", "dq[b, s0:s0 + 256, hi, :] = scale * (ds @ kb)", "dq[b, s0:s0 + 256, hi, :] = ds @ kb"),
    ("chunked form drops D", "        dp -= d\n", "        dp -= 0.0 * d\n"),
    ("chunked key gradients overwritten per chunk", "dk[bi, :lk, hi, :] += dkc", "dk[bi, :lk, hi, :] = dkc"),
    ("chunked dV uses dS", "return scale * (dp @ kb), scale * (dp.T @ qc), p.T @ gc",
     "return scale * (dp @ kb), scale * (dp.T @ qc), dp.T @ gc"),
    ("chunked form drops a ragged last chunk", "starts = list(range(0, L, chunk))",
     "starts = list(range(0, L - chunk + 1, chunk))"),
    ("chunked dK drops the scale", "return scale * (dp @ kb), scale * (dp.T @ qc), p.T @ gc",
     "return scale * (dp @ kb), (dp.T @ qc), p.T @ gc"),
    ("varlen backward key rows shifted", "kb, vb = k[k0:k1, h, :], v[k0:k1, h, :]",
     "kb, vb = k[k0:k1, h, :], v[q0:q0 + (k1 - k0), h, :]"),
]


def _stage(dst, mutant=None):
    """Copy the oracle, the input module and the pin tests into dst; apply one edit."""
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "hvinputs.py"), dst)
    tdir = os.path.join(dst, "tests")
    os.makedirs(tdir)
    for f in os.listdir(os.path.join(ROOT, "tests")):
        if f.startswith("test_oracle_") and f.endswith(".py") and f != "test_oracle_mutants.py":
            shutil.copy(os.path.join(ROOT, "tests", f), tdir)
    shutil.copy(os.path.join(ROOT, "tests", "conftest.py"), tdir)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tdir, "golden"))
    if mutant is not None:
        _, old, new = mutant
        path = os.path.join(dst, ORACLE)
        src = open(path).read()
        assert src.count(old) == 1, f"mutant {mutant[0]!r} does not apply exactly once"
        open(path, "w").write(src.replace(old, new))


def _run_pins(dst) -> int:
    env = dict(os.environ, PYTHONPATH=dst, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1",
               OPENBLAS_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests"], cwd=dst, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def test_every_mutant_fails_a_pin(tmp_path):
    base = tmp_path / "clean"
    _stage(str(base))
    assert _run_pins(str(base)) == 0, "the unmutated oracle must pass its pins"

    def one(i):
        d = tmp_path / f"m{i}"
        _stage(str(d), MUTANTS[i])
        return _run_pins(str(d))

    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        codes = list(pool.map(one, range(len(MUTANTS))))
    survivors = [MUTANTS[i][0] for i, c in enumerate(codes) if c == 0]
    assert not survivors, f"mutants that no pin catches: {survivors}"
    # a failing pin run exits with 1; anything else (2: an import or collection
    # error) would mean the mutant broke the module rather than a pin caught it
    broken = [MUTANTS[i][0] for i, c in enumerate(codes) if c not in (0, 1)]
    assert not broken, f"mutants that break collection instead of a pin: {broken}"
