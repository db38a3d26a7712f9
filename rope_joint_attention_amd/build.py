"""Build libhvattn.so in-tree with hipcc for gfx950.

    python -m rope_joint_attention_amd.build               # lib/libhvattn.so
    python -m rope_joint_attention_amd.build --host-sanitizers OUT.so

Compiles every HIP source under csrc/ into one shared library next to this
file (``lib/libhvattn.so``).  Always recompiles.

--host-sanitizers builds the same sources with AddressSanitizer and
UndefinedBehaviorSanitizer on the host code only (argument validation, launch
set-up); the device code is compiled exactly as in the normal build.  The
result needs the sanitizer runtime preloaded into the process
(LD_PRELOAD=<ROCm llvm>/lib/clang/<v>/lib/linux/libclang_rt.asan-x86_64.so)
and is selected for the Python binding with HVATTN_LIBRARY=OUT.so.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libhvattn.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-mcode-object-version=5",
    # no packed fp32 VALU ops in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMAs accumulate in VGPRs: the dK/dV kernel keeps its K/V operands in
    # AGPRs and its score accumulators in VGPRs, where the softmax reads them
    # (the other kernels' code is the same either way)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
]

# Flags for one source only.  attn_fwd.hip: its work-counter atomic is taken by
# one lane, and without the atomic optimizer's lane scan the result is not
# waited for right away, so the round trip for the next block id overlaps the
# block's first loads (the backward kernels keep the default, which leaves
# their register allocation as it is).
FILE_FLAGS = {
    "attn_fwd.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
}


# host-only instrumentation: every sanitizer flag applies to the host pass
HOST_SANITIZER_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                        "-Xarch_host -fno-sanitize-recover=undefined "
                        "-Xarch_host -fno-omit-frame-pointer -Xarch_host -g").split()


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of the ROCm clang (for LD_PRELOAD)."""
    pats = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not pats:
        raise RuntimeError("ROCm clang's AddressSanitizer runtime not found")
    return sorted(pats)[-1]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (needs ROCm)")


def _run(cmd, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = True, out: str = LIB, host_sanitizers: bool = False) -> str:
    """Compile every source to an object (in parallel, each with its own
    flags), then link the shared library."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    extra = HOST_SANITIZER_FLAGS if host_sanitizers else []
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    common = [f for f in HIPCC_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="hvattn_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in sources]
        cmds = [[hipcc(), *common, *FILE_FLAGS.get(os.path.basename(src), []), *extra, *inc,
                 "-c", "-o", obj, src] for src, obj in zip(sources, objs)]
        with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as pool:
            list(pool.map(lambda c: _run(c, verbose), cmds))
        tmp = out + ".tmp"
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs], verbose)
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--host-sanitizers":
        print(build(out=os.path.abspath(sys.argv[2]), host_sanitizers=True))
    else:
        print(build())
