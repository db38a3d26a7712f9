"""The host side of libhvattn under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with both sanitizers on its host code (argument
validation, segment tables, launch set-up; the device code is compiled as
usual) and every C-ABI check of test_abi_cpu.py runs against that build in a
child process with the sanitizer runtime preloaded.  Any report fails the
test.  Two control cases show that the harness reports what it should: a
planted heap over-read and a planted out-of-range shift, each in a throwaway
C function built the same way (never in the library).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/lib/llvm/bin/clang"

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="needs hipcc")


def _env(lib):
    from rope_joint_attention_amd.build import asan_runtime

    return dict(os.environ, LD_PRELOAD=asan_runtime(), HVATTN_LIBRARY=lib,
                ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=23",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=24",
                PYTHONDONTWRITEBYTECODE="1")


def _reported(text: str) -> bool:
    return "ERROR: AddressSanitizer" in text or "runtime error:" in text


def test_control_cases_are_reported(tmp_path):
    src = tmp_path / "planted.c"
    src.write_text(
        "#include <stdlib.h>\n"
        "int over_read(int n) { int* a = malloc(n * sizeof(int)); for (int i = 0; i < n; ++i) a[i] = i;\n"
        "  int s = a[n]; free(a); return s; }\n"
        "int bad_shift(int s) { return 1 << s; }\n")
    so = tmp_path / "libplanted.so"
    subprocess.run([CLANG, "-shared", "-fPIC", "-O1", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-o", str(so), str(src)], check=True)
    for call in ("over_read(4)", "bad_shift(40)"):
        code = f"import ctypes; lib = ctypes.CDLL({str(so)!r}); lib.{call}"
        r = subprocess.run([sys.executable, "-c", code], env=_env(""), capture_output=True,
                           text=True, timeout=120)
        assert r.returncode != 0 and _reported(r.stderr), (call, r.returncode, r.stderr[-2000:])


@pytest.mark.timeout(600)
def test_abi_checks_clean_under_host_sanitizers(tmp_path):
    from rope_joint_attention_amd.build import build

    lib = build(verbose=False, out=str(tmp_path / "libhvattn_hostsan.so"), host_sanitizers=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=_env(lib), capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert not _reported(out), out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout and "skipped" not in r.stdout.splitlines()[-1], r.stdout[-2000:]
