"""include/hvattn.h is a plain C header: a C99 program includes it with no HIP
or C++ headers, links libhvattn.so and calls the host-only and validation
paths on the CPU.

* the header compiles under gcc -std=c99 -pedantic -Wall -Werror;
* hv_token_grid returns the notes page's worked example (section 4:
  544x960x17 -> latent 5x68x120, token grid 5x34x60, 10200 tokens) and
  rejects a frame count that is not 4k+1;
* hv_joint_attention_fwd with a NULL q and an empty call report
  HV_ERR_INVALID_ARG and HV_OK before any HIP call; hv_status_string never
  returns NULL.
"""
import os
import shutil
import subprocess

import pytest

import rope_joint_attention_amd as hv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = [
    pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc"),
    pytest.mark.skipif(not os.path.exists(hv.library_path()), reason="libhvattn.so not built"),
]

PROGRAM = r"""
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include "hvattn.h"

/* 16-byte aligned addresses that are never dereferenced: every call below is
   decided by the host-side checks */
#define FAKE(i) ((hv_bf16*)(uintptr_t)((1ULL << 40) + (uint64_t)(i) * (1ULL << 30)))

int main(void) {
  hv_grid g;
  hv_layout lay;
  int st = hv_token_grid(17, 544, 960, &g);
  printf("grid %d %d %d %d %d %d %d %lld\n", st, g.t_lat, g.h_lat, g.w_lat, g.gt, g.gh, g.gw,
         (long long)g.n_video);
  printf("bad_frames %d\n", hv_token_grid(16, 544, 960, &g));
  memset(&lay, 0, sizeof lay);
  lay.batch = 1; lay.seq_len = 64; lay.heads = HV_HEADS; lay.head_dim = HV_HEAD_DIM;
  lay.stride_b = 64LL * HV_HEADS * HV_HEAD_DIM; lay.stride_l = HV_HEADS * HV_HEAD_DIM;
  printf("null_q %d\n", hv_joint_attention_fwd(NULL, FAKE(1), FAKE(2), NULL, FAKE(3), &lay, 64,
                                                 0.0f, NULL, 0, NULL));
  lay.batch = 0;
  printf("empty %d\n", hv_joint_attention_fwd(FAKE(0), FAKE(1), FAKE(2), NULL, FAKE(3), &lay, 0,
                                                0.0f, NULL, 0, NULL));
  printf("strings %d\n", hv_status_string(HV_ERR_HIP) != NULL && hv_status_string(12345) != NULL);
  printf("version %d\n", hv_version() > 0);
  return 0;
}
"""


def test_header_is_c99_and_links(tmp_path):
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(hv.library_path())
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
           "-L", libdir, "-l:" + os.path.basename(hv.library_path()), "-Wl,-rpath," + libdir]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    lines = dict(ln.split(" ", 1) for ln in run.stdout.strip().splitlines())
    assert lines["grid"] == "0 5 68 120 5 34 60 10200"
    assert int(lines["bad_frames"]) == hv.HV_ERR_INVALID_ARG
    assert int(lines["null_q"]) == hv.HV_ERR_INVALID_ARG
    assert int(lines["empty"]) == hv.HV_OK
    assert lines["strings"] == "1" and lines["version"] == "1"
