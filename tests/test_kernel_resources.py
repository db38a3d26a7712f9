"""Register budget of every HIP kernel, from the compiler's own report.

Each source under csrc/ is compiled for gfx950 (device code only, the
library's flags) with -Rpass-analysis=kernel-resource-usage, and the report
is checked against the budget the kernels are designed for: no scratch
memory at all (no VGPR spills, no stack), the attention kernels at their
occupancy (two waves per SIMD for the 8-wave forward and the dQ kernel, one
for the 4-wave forward of small calls and for dK/dV),
and at most a bounded number of SGPRs spilled (those go to VGPR lanes, never
to memory).  A change that starts spilling inside the key loop shows up here
before it shows up as a slower kernel.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rope_joint_attention_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="needs hipcc")

# kernel (demangled-name fragment) -> (waves per SIMD, most SGPRs spilled)
BUDGET = {
    "attn_fwd_kernelILb1ELi8": (2, 72),
    "attn_fwd_kernelILb0ELi4": (1, 80),   # before the 8-wave entry: matched by fragment
    "attn_fwd_kernelILb0ELi8": (2, 64),
    "attn_bwd_delta_kernel": (None, 0),
    "attn_bwd_dkdv_kernel": (1, 8),
    "attn_bwd_dq_kernel": (2, 8),
    "v_pack_kernel": (None, 0),
    "qknorm_rope3d_kernel": (None, 0),   # before rope3d_kernel: names are matched by fragment
    "rope3d_kernel": (None, 0),
    "attn_merge_kernel": (None, 0),
}


def resource_report(src):
    from rope_joint_attention_amd.build import FILE_FLAGS, HIPCC_FLAGS, hipcc

    flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")] + FILE_FLAGS.get(src, [])
    cmd = [hipcc(), *flags, "--cuda-device-only", "-c", "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark: \s*([A-Za-z /\[\]]+?): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return kernels


def test_kernels_stay_within_their_register_budget():
    sources = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip") and f != "hvattn_api.hip")
    with ThreadPoolExecutor(max_workers=min(8, len(sources))) as pool:
        reports = dict(zip(sources, pool.map(resource_report, sources)))
    seen = set()
    for src, kernels in reports.items():
        for name, r in kernels.items():
            key = next((k for k in BUDGET if k in name), None)
            assert key is not None, f"{src}: kernel {name} has no budget entry"
            seen.add(key)
            waves, sgpr_spill = BUDGET[key]
            assert r["ScratchSize [bytes/lane]"] == 0, (name, r)
            assert r["VGPRs Spill"] == 0, (name, r)
            assert r["SGPRs Spill"] <= sgpr_spill, (name, r)
            if waves is not None:
                assert r["Occupancy [waves/SIMD]"] >= waves, (name, r)
    assert seen == set(BUDGET), set(BUDGET) - seen
