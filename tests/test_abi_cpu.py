"""C-ABI checks that need no GPU.

* libhvattn.so loads and exports every function include/hvattn.h declares,
  and imports no HIP allocation, copy, memset or synchronisation function;
* hv_token_grid (host-only) agrees with the printed values and the oracle;
* every host-side validation path of hv_rope3d_apply and
  hv_joint_attention_fwd returns its documented status without touching
  memory (fake, never-dereferenced device addresses are passed; the
  library validates everything before its first HIP call).
"""
import ctypes
import json
import os
import re

import pytest

import rope_joint_attention_amd as hv
from oracle import token_grid as oracle_grid

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hvattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(hv.library_path()),
                                reason="libhvattn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hv_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    lib = hv.load_library()
    names = declared_functions()
    assert set(names) >= {"hv_token_grid", "hv_rope3d_apply", "hv_joint_attention_fwd",
                          "hv_status_string", "hv_version"}
    for n in names:
        assert hasattr(lib, n), n
    # and nothing else hv_* is exported that the header does not declare
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", hv.library_path()], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r" T (hv_[a-z0-9_]+)$", out, flags=re.M)))
    assert exported == names


# The HIP runtime functions the library may import: kernel registration and
# launch, the device query of the forward's CU count, the scratch address of
# the allocation-free backward, and error reporting.  No allocation, no copy
# or memset (which a caller's graph capture would record as separate nodes),
# no synchronisation: the calls only enqueue kernels on the caller's stream.
ALLOWED_HIP_IMPORTS = {
    "__hipPopCallConfiguration", "__hipPushCallConfiguration", "__hipRegisterFatBinary",
    "__hipRegisterFunction", "__hipRegisterVar", "__hipUnregisterFatBinary",
    "hipLaunchKernel", "hipGetDevice", "hipDeviceGetAttribute", "hipGetSymbolAddress",
    "hipGetLastError",
}


def test_library_imports_no_allocation_copy_or_synchronisation():
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", hv.library_path()], capture_output=True,
                         text=True, check=True).stdout
    imported = {m.split("@")[0] for m in re.findall(r"\bU (\S+)", out)}
    hip = {n for n in imported if "hip" in n.lower()}
    assert hip, "no HIP imports found: nm output not understood"
    assert hip <= ALLOWED_HIP_IMPORTS, sorted(hip - ALLOWED_HIP_IMPORTS)
    banned = re.compile(r"malloc|free|memset|memcpy|synchron|hostregister", re.I)
    assert not [n for n in hip if banned.search(n)]


def test_status_strings():
    for st in (0, -1, -2, -3, 7):
        s = hv.hv_status_string(st)
        assert isinstance(s, str) and s
    assert "INVALID" in hv.hv_status_string(-1)
    assert hv.load_library().hv_version() >= 10000


GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "token_grid.json")))


def test_token_grid_printed_values():
    for c in GOLDEN["cases"]:
        g = hv.hv_token_grid(c["frames"], c["height"], c["width"])
        if "n_video" in c:
            assert g.n_video == c["n_video"]
        if "latent" in c:
            assert (g.t_lat, g.h_lat, g.w_lat) == tuple(c["latent"])
        if "token_grid" in c:
            assert (g.gt, g.gh, g.gw) == tuple(c["token_grid"])


@pytest.mark.parametrize("fhw,n", [((129, 1104, 832), 118404), ((129, 624, 832), 66924),
                                   ((129, 720, 720), 66825), ((129, 960, 960), 118800)])
def test_token_grid_hand_worked_counts(fhw, n):
    # 33 x (H/16) x (W/16), worked by hand: 33*69*52, 33*39*52, 33*45*45, 33*60*60
    assert hv.hv_token_grid(*fhw).n_video == n


@pytest.mark.parametrize("fhw", [(f, h, w) for f in (1, 5, 17, 33, 65, 129, 257)
                                 for h, w in ((256, 256), (544, 960), (720, 1280), (1104, 832), (16, 16), (960, 960))])
def test_token_grid_matches_oracle(fhw):
    g = hv.hv_token_grid(*fhw)
    o = oracle_grid(*fhw)
    for f in ("t_lat", "h_lat", "w_lat", "gt", "gh", "gw", "n_video"):
        assert getattr(g, f) == getattr(o, f), f


@pytest.mark.parametrize("fhw", GOLDEN["rejected"]["cases"] + [[-3, 544, 960], [17, 544, -16], [2, 16, 16]])
def test_token_grid_rejects(fhw):
    with pytest.raises(hv.HvError) as ei:
        hv.hv_token_grid(*fhw)
    assert ei.value.status == hv.HV_ERR_INVALID_ARG


def test_token_grid_null_out():
    lib = hv.load_library()
    assert lib.hv_token_grid(17, 544, 960, None) == hv.HV_ERR_INVALID_ARG


# ---------------------------------------------------------------- validation
FAKE = 1 << 40           # 16-byte aligned, never dereferenced
SEP = 1 << 34            # far apart so default tensors never overlap


def layout(batch=1, seq=300, heads=24, dim=128, sb=None, sl=3072):
    lay = hv._Layout()
    lay.batch, lay.seq_len, lay.heads, lay.head_dim = batch, seq, heads, dim
    lay.stride_l = sl
    lay.stride_b = seq * sl if sb is None else sb
    return lay


def grid(F=5, H=64, W=80):
    return hv.hv_token_grid(F, H, W)._c()   # 2 x 4 x 5 = 40 video tokens


def rope(q=FAKE, k=FAKE + SEP, lay=None, g=None, theta=10000.0):
    lib = hv.load_library()
    lay = layout() if lay is None else lay
    g = grid() if g is None else g
    return lib.hv_rope3d_apply(q, k, ctypes.byref(lay) if lay is not False else None,
                               ctypes.byref(g) if g is not False else None, theta, None)


def attn(q=FAKE, k=FAKE + SEP, v=FAKE + 2 * SEP, out=FAKE + 3 * SEP, valid=(10,), lay=None,
         n_video=40, scale=0.0, ws=None, ws_bytes=0):
    lib = hv.load_library()
    lay = layout() if lay is None else lay
    arr = None if valid is None else (ctypes.c_int32 * max(1, len(valid)))(*valid)
    return lib.hv_joint_attention_fwd(q, k, v, arr, out, ctypes.byref(lay) if lay is not False else None,
                                      n_video, scale, ws, ws_bytes, None)


E, U = hv.HV_ERR_INVALID_ARG, hv.HV_ERR_UNSUPPORTED


@pytest.mark.parametrize("kwargs,expect", [
    (dict(q=0), E), (dict(k=0), E), (dict(lay=False), E), (dict(g=False), E),
    (dict(q=FAKE + 2), E), (dict(k=FAKE + SEP + 8), E),
    (dict(k=FAKE + 3072 * 2), E),                         # k overlaps q
    (dict(theta=0.0), E), (dict(theta=-1.0), E), (dict(theta=float("nan")), E), (dict(theta=float("inf")), E),
    (dict(lay=layout(heads=16)), U), (dict(lay=layout(dim=64)), U),
    (dict(lay=layout(batch=65)), U),
    (dict(lay=layout(seq=(1 << 24) + 1)), U),
    (dict(lay=layout(batch=-1)), E), (dict(lay=layout(seq=-5)), E),
    (dict(lay=layout(sl=3000)), E), (dict(lay=layout(sl=3076)), E),
    (dict(lay=layout(sl=(1 << 24) + 8)), U),             # token stride beyond the 32-bit tile offsets
    (dict(lay=layout(batch=2, sb=3072 * 10)), E),         # batch stride too small
    (dict(lay=layout(seq=39)), E),                        # fewer rows than video tokens
])
def test_rope_validation(kwargs, expect):
    assert rope(**kwargs) == expect


def test_rope_inconsistent_grid():
    g = grid()
    g.n_video = 41
    assert rope(g=g) == E
    g = grid()
    g.gw = 0
    assert rope(g=g) == E


@pytest.mark.parametrize("kwargs,expect", [
    (dict(q=0), E), (dict(k=0), E), (dict(v=0), E), (dict(out=0), E), (dict(lay=False), E),
    (dict(v=FAKE + 2 * SEP + 4), E), (dict(out=FAKE + 3 * SEP + 2), E),
    (dict(out=FAKE + 100 * 3072 * 2), E),                 # out overlaps q
    (dict(out=FAKE + SEP - 64), E),                       # out overlaps the start of k
    (dict(out=FAKE + 2 * SEP + 299 * 3072 * 2), E),       # out overlaps the last row of v
    (dict(valid=(-1,)), E), (dict(valid=(261,)), E),      # text capacity is 300 - 40 = 260
    (dict(n_video=-1), E), (dict(n_video=301), E),
    (dict(n_video=0, valid=(0,)), E),                     # no valid key
    (dict(lay=layout(heads=32)), U), (dict(lay=layout(dim=256)), U),
    (dict(lay=layout(batch=65), valid=None), U),
    (dict(lay=layout(sl=3080 + 4)), E),
    (dict(lay=layout(batch=2, sb=3072 * 299), valid=(1, 1)), E),
])
def test_attention_validation(kwargs, expect):
    assert attn(**kwargs) == expect


def test_attention_second_batch_entry_checked():
    assert attn(lay=layout(batch=3, seq=300), valid=(10, 10, 999)) == E
    assert attn(lay=layout(batch=3, seq=300), valid=(10, -2, 5)) == E


def test_empty_calls_are_noops():
    # batch 0 or seq 0: nothing to compute, no launch (so no GPU needed)
    assert attn(lay=layout(batch=0), valid=None, n_video=0) == hv.HV_OK
    assert attn(lay=layout(seq=0, sb=0), valid=(0,), n_video=0) == hv.HV_OK
    assert rope(lay=layout(batch=0)) == hv.HV_OK


@pytest.mark.parametrize("delta_elems,sl,batch,sb", [
    (1024, 9216, 1, None),        # rows of k start 1024 channels into q's rows
    (7000, 9216, 1, None),        # k's row would run into q's next row
    (9216 * 5, 9216, 1, None),    # same rows, five tokens later
    (3072, 9216, 2, 9216 * 300 + 8),  # batch stride not a multiple of the token stride
])
def test_interleaved_views_that_alias_are_rejected(delta_elems, sl, batch, sb):
    lay = layout(batch=batch, sl=sl, sb=sb)
    assert rope(k=FAKE + 2 * delta_elems, lay=lay) == E
    valid = (10,) * batch
    assert attn(out=FAKE + SEP + 2 * delta_elems, lay=lay, valid=valid) == E


def test_odd_byte_offset_counts_as_aliasing():
    lay = layout(sl=9216)
    # 16-byte aligned but an odd element offset is impossible; an unaligned
    # pointer is rejected first, by the alignment rule
    assert rope(k=FAKE + 2 * 3072 + 1, lay=lay) == E


# ---------------------------------------------------- QK-norm + RoPE prologue
GQ, GK = FAKE + 4 * SEP, FAKE + 4 * SEP + 256


def qknorm(q=FAKE, k=FAKE + SEP, lay=None, g=None, theta=10000.0, gq=GQ, gk=GK, gqt=None, gkt=None,
           eps=1e-6):
    lib = hv.load_library()
    lay = layout() if lay is None else lay
    g = grid() if g is None else g
    return lib.hv_qk_norm_rope3d_apply(q, k, ctypes.byref(lay) if lay is not False else None,
                                       ctypes.byref(g) if g is not False else None, theta,
                                       gq, gk, gqt, gkt, eps, None)


@pytest.mark.parametrize("kwargs,expect", [
    (dict(q=0), E), (dict(k=0), E), (dict(gq=0), E), (dict(gk=0), E),
    (dict(lay=False), E), (dict(g=False), E),
    (dict(q=FAKE + 2), E), (dict(gq=GQ + 8), E), (dict(gk=GK + 2), E),
    (dict(gqt=GQ + 4 + 512), E), (dict(gkt=GK + 8 + 512), E),
    (dict(k=FAKE + 3072 * 2), E),                         # k overlaps q
    (dict(gq=FAKE + 160 * 3072 * 2), E),                  # weight inside q
    (dict(gk=FAKE + SEP + 299 * 3072 * 2 + 128), E),      # weight inside k's last row
    (dict(gqt=FAKE + SEP - 128), E),                      # text weight straddles k's start
    (dict(theta=0.0), E), (dict(theta=float("nan")), E),
    (dict(eps=-1e-6), E), (dict(eps=float("nan")), E), (dict(eps=float("inf")), E),
    (dict(lay=layout(heads=16)), U), (dict(lay=layout(dim=64)), U), (dict(lay=layout(batch=65)), U),
    (dict(lay=layout(batch=-1)), E), (dict(lay=layout(sl=3076)), E),
    (dict(lay=layout(seq=39)), E),                        # fewer rows than video tokens
])
def test_qknorm_validation(kwargs, expect):
    assert qknorm(**kwargs) == expect


def test_qknorm_weights_may_alias_each_other_and_empty_calls_are_noops():
    # shared weights (text = video, q = k) pass validation; batch 0 launches nothing
    assert qknorm(gk=GQ, gqt=GQ, gkt=GQ, lay=layout(batch=0)) == hv.HV_OK
    assert qknorm(lay=layout(seq=0, sb=0), g=grid(1, 16, 16)) == E   # 1 video token > 0 rows
    assert qknorm(lay=layout(batch=0), eps=0.0) == hv.HV_OK


def test_qknorm_inconsistent_grid():
    g = grid()
    g.n_video = 39
    assert qknorm(g=g) == E


# --------------------------------------- attention with LSE, merge, varlen
LSE = FAKE + 8 * SEP


def attn_lse(q=FAKE, k=FAKE + SEP, v=FAKE + 2 * SEP, out=FAKE + 3 * SEP, lse=LSE, valid=None,
             qlay=None, kvlay=None, scale=0.0, ws=None, ws_bytes=0):
    lib = hv.load_library()
    qlay = layout(seq=200) if qlay is None else qlay
    kvlay = layout(seq=300) if kvlay is None else kvlay
    arr = None if valid is None else (ctypes.c_int32 * max(1, len(valid)))(*valid)
    return lib.hv_attention_fwd_lse(q, ctypes.byref(qlay) if qlay is not False else None, k, v,
                                    ctypes.byref(kvlay) if kvlay is not False else None, arr, out,
                                    lse, scale, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,expect", [
    (dict(q=0), E), (dict(k=0), E), (dict(v=0), E), (dict(out=0), E),
    (dict(qlay=False), E), (dict(kvlay=False), E),
    (dict(qlay=layout(batch=2, seq=200)), E),                 # batch mismatch
    (dict(valid=(0,)), E), (dict(valid=(301,)), E), (dict(valid=(-4,)), E),
    (dict(lse=LSE + 2), E),                                   # lse alignment
    (dict(out=FAKE + 2 * SEP + 4096), E),                     # out inside v (other layout)
    (dict(out=FAKE + 100 * 3072 * 2), E),                     # out inside q
    (dict(lse=FAKE + SEP + 64), E),                           # lse inside k
    (dict(lse=FAKE + 3 * SEP + 8), E),                        # lse inside out
    (dict(qlay=layout(seq=200, heads=8)), U), (dict(kvlay=layout(seq=300, dim=64)), U),
    (dict(kvlay=layout(seq=300, sl=3076)), E),
])
def test_attention_lse_validation(kwargs, expect):
    assert attn_lse(**kwargs) == expect


def test_attention_lse_empty_and_optional_lse():
    assert attn_lse(qlay=layout(batch=0, seq=200), kvlay=layout(batch=0, seq=300)) == hv.HV_OK
    assert attn_lse(qlay=layout(seq=0, sb=0)) == hv.HV_OK
    # lse = NULL passes validation as well (empty call: nothing launched)
    assert attn_lse(lse=None, qlay=layout(seq=0, sb=0)) == hv.HV_OK


def merge(outs=None, lses=None, n=None, out=FAKE + 3 * SEP, lse_out=FAKE + 9 * SEP, lay=None):
    lib = hv.load_library()
    outs = [FAKE, FAKE + SEP] if outs is None else outs
    lses = [FAKE + 6 * SEP, FAKE + 7 * SEP] if lses is None else lses
    n = len(outs) if n is None else n
    oa = (ctypes.c_void_p * max(1, len(outs)))(*outs)
    la = (ctypes.c_void_p * max(1, len(lses)))(*lses)
    lay = layout() if lay is None else lay
    return lib.hv_attention_merge(oa, la, n, out, lse_out, ctypes.byref(lay), None)


@pytest.mark.parametrize("kwargs,expect", [
    (dict(n=0), E), (dict(outs=[FAKE] * 17, lses=[FAKE + 6 * SEP] * 17), E),
    (dict(outs=[FAKE, 0]), E), (dict(lses=[FAKE + 6 * SEP, 0]), E), (dict(out=0), E),
    (dict(outs=[FAKE, FAKE + SEP + 8]), E), (dict(lses=[FAKE + 6 * SEP, FAKE + 7 * SEP + 2]), E),
    (dict(out=FAKE + 3 * SEP + 4), E), (dict(lse_out=FAKE + 9 * SEP + 1), E),
    (dict(out=FAKE + SEP), E),                                # out is a partial output
    (dict(lse_out=FAKE + 7 * SEP), E),                        # lse_out is a partial lse
    (dict(lse_out=FAKE + 3 * SEP + 64), E),                   # lse_out inside out
    (dict(lses=[FAKE + 3 * SEP + 128, FAKE + 7 * SEP]), E),   # an input lse inside out
    (dict(lay=layout(heads=12)), U),
])
def test_merge_validation(kwargs, expect):
    assert merge(**kwargs) == expect


def test_merge_accepts_16_parts_and_null_lse_out_when_empty():
    outs = [FAKE + i * (1 << 30) for i in range(16)]
    lses = [FAKE + 12 * SEP + i * (1 << 30) for i in range(16)]
    assert merge(outs=outs, lses=lses, out=FAKE + 30 * SEP, lse_out=None,
                 lay=layout(batch=0)) == hv.HV_OK


def varlen(cq=(0, 100, 300), ck=None, n=None, q=FAKE, k=FAKE + SEP, v=FAKE + 2 * SEP,
           out=FAKE + 3 * SEP, lse=LSE, lay=None, ws=None, ws_bytes=0):
    lib = hv.load_library()
    ck = cq if ck is None else ck
    n = len(cq) - 1 if n is None else n
    aq = (ctypes.c_int32 * len(cq))(*cq)
    ak = (ctypes.c_int32 * len(ck))(*ck)
    lay = layout() if lay is None else lay
    return lib.hv_joint_attention_varlen_fwd(q, k, v, aq, ak, n, out, lse, ctypes.byref(lay), 0.0,
                                             ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,expect", [
    (dict(q=0), E), (dict(k=0), E), (dict(v=0), E), (dict(out=0), E),
    (dict(n=0), E), (dict(n=65, cq=tuple(range(66)), ck=tuple(range(66))), E),
    (dict(cq=(0, 100, 301)), E),                              # past the packed rows
    (dict(cq=(0, 120, 100)), E),                              # decreasing
    (dict(cq=(-1, 100, 300)), E),
    (dict(cq=(0, 100, 300), ck=(0, 100, 100)), E),            # queries without keys
    (dict(lay=layout(batch=2, sb=300 * 3072)), E),            # packed layout has batch 1
    (dict(lse=LSE + 2), E), (dict(lse=FAKE + 40), E),         # lse inside q
    (dict(out=FAKE + SEP + 3072 * 2 * 5), E),                 # out inside k
    (dict(lay=layout(heads=12)), U),
])
def test_varlen_validation(kwargs, expect):
    assert varlen(**kwargs) == expect


def test_varlen_empty_segments_are_valid():
    # all-empty segments: nothing to launch
    assert varlen(cq=(0, 0, 0), ck=(0, 0, 5)) == hv.HV_OK
    assert varlen(cq=(0, 0), ck=(0, 0), lay=layout(seq=0, sb=0)) == hv.HV_OK


# ------------------------------------------------------------ backward
def bwd(q=FAKE, k=FAKE + SEP, v=FAKE + 2 * SEP, o=FAKE + 3 * SEP, g=FAKE + 4 * SEP, lse=LSE,
        valid=(10,), n_video=40, dq=FAKE + 10 * SEP, dk=FAKE + 11 * SEP, dv=FAKE + 12 * SEP,
        delta=FAKE + 13 * SEP, lay=None):
    lib = hv.load_library()
    lay = layout() if lay is None else lay
    arr = None if valid is None else (ctypes.c_int32 * max(1, len(valid)))(*valid)
    return lib.hv_joint_attention_bwd(q, k, v, o, g, lse, arr, n_video, dq, dk, dv, delta,
                                      ctypes.byref(lay) if lay is not False else None, 0.0, None)


@pytest.mark.parametrize("kwargs,expect", [
    (dict(q=0), E), (dict(k=0), E), (dict(v=0), E), (dict(o=0), E), (dict(g=0), E),
    (dict(lse=0), E), (dict(dq=0), E), (dict(dk=0), E), (dict(dv=0), E), (dict(delta=0), E),
    (dict(lay=False), E), (dict(dq=FAKE + 10 * SEP + 2), E), (dict(lse=LSE + 1), E),
    (dict(delta=FAKE + 13 * SEP + 2), E),
    (dict(dq=FAKE + 100 * 3072 * 2), E),                  # dq inside q
    (dict(dk=FAKE + 10 * SEP + 64 * 3072 * 2), E),        # dk inside dq
    (dict(dv=FAKE + 4 * SEP), E),                         # dv is dout
    (dict(delta=LSE + 64), E),                            # delta inside lse
    (dict(delta=FAKE + 12 * SEP + 128), E),               # delta inside dv
    (dict(lse=FAKE + 2 * SEP + 256), E),                  # lse inside v
    (dict(valid=(-1,)), E), (dict(valid=(261,)), E), (dict(n_video=0, valid=(0,)), E),
    (dict(n_video=301), E),
    (dict(lay=layout(heads=8)), U), (dict(lay=layout(batch=65), valid=None), U),
])
def test_backward_validation(kwargs, expect):
    assert bwd(**kwargs) == expect


D_BYTES = 2 * 24 * 300 * 4   # -D and -lse/scale of the default layout; 256 bytes of counters follow


def test_backward_delta_includes_the_counters():
    # (arguments that pass every check would launch on these fake pointers,
    # so only refusals are asked for here)
    assert bwd(delta=LSE - D_BYTES) == E                  # counters would overwrite lse
    assert bwd(delta=LSE - D_BYTES - 252) == E
    assert bwd(lse=FAKE + 13 * SEP + D_BYTES + 128) == E
    assert bwd(dq=FAKE + 13 * SEP + D_BYTES + 240, dk=FAKE + 11 * SEP) == E
    assert varlen_bwd(delta=LSE - D_BYTES) == E


def test_backward_empty_call():
    assert bwd(lay=layout(batch=0), valid=None, n_video=0) == hv.HV_OK


def bwd_noalloc(q=FAKE, k=FAKE + SEP, v=FAKE + 2 * SEP, o=FAKE + 3 * SEP, g=FAKE + 4 * SEP, lse=LSE,
                valid=(10,), n_video=40, dq=FAKE + 10 * SEP, dk=FAKE + 11 * SEP, dv=FAKE + 12 * SEP,
                lay=None):
    lib = hv.load_library()
    lay = layout() if lay is None else lay
    arr = None if valid is None else (ctypes.c_int32 * max(1, len(valid)))(*valid)
    return lib.hv_joint_attention_bwd_noalloc(q, k, v, o, g, lse, arr, n_video, dq, dk, dv,
                                              ctypes.byref(lay) if lay is not False else None,
                                              0.0, None)


NOALLOC_ROWS = (hv.HV_NOALLOC_BWD_SCRATCH_BYTES - 256) // (2 * 24 * 4)   # batch * seq_len limit


@pytest.mark.parametrize("kwargs,expect", [
    (dict(q=0), E), (dict(k=0), E), (dict(v=0), E), (dict(o=0), E), (dict(g=0), E),
    (dict(lse=0), E), (dict(dq=0), E), (dict(dk=0), E), (dict(dv=0), E),
    (dict(lay=False), E), (dict(dq=FAKE + 10 * SEP + 2), E), (dict(lse=LSE + 1), E),
    (dict(dq=FAKE + 100 * 3072 * 2), E),                  # dq inside q
    (dict(dv=FAKE + 4 * SEP), E),                         # dv is dout
    (dict(lse=FAKE + 2 * SEP + 256), E),                  # lse inside v
    (dict(valid=(-1,)), E), (dict(valid=(261,)), E), (dict(n_video=0, valid=(0,)), E),
    (dict(n_video=301), E),
    (dict(lay=layout(heads=8)), U), (dict(lay=layout(batch=65), valid=None), U),
    # over the static scratch: one row more than it holds, in one or two entries
    (dict(lay=layout(seq=NOALLOC_ROWS + 1), n_video=NOALLOC_ROWS + 1 - 256, valid=(256,)), U),
    (dict(lay=layout(batch=2, seq=NOALLOC_ROWS // 2 + 1, sb=(NOALLOC_ROWS // 2 + 1) * 3072),
          n_video=NOALLOC_ROWS // 2 + 1 - 256, valid=(256, 3)), U),
])
def test_backward_noalloc_validation(kwargs, expect):
    assert bwd_noalloc(**kwargs) == expect


def test_backward_noalloc_limit_and_empty_call():
    assert NOALLOC_ROWS == 174762                          # 720x1280x129 (119056 rows) fits
    assert bwd_noalloc(lay=layout(batch=0), valid=None, n_video=0) == hv.HV_OK
    assert bwd_noalloc(lay=layout(batch=0), valid=None, n_video=301) == E


def varlen_bwd(cq=(0, 100, 300), ck=None, n=None, lay=None, **kw):
    lib = hv.load_library()
    ck = cq if ck is None else ck
    n = len(cq) - 1 if n is None else n
    aq = (ctypes.c_int32 * len(cq))(*cq)
    ak = (ctypes.c_int32 * len(ck))(*ck)
    lay = layout() if lay is None else lay
    a = dict(q=FAKE, k=FAKE + SEP, v=FAKE + 2 * SEP, o=FAKE + 3 * SEP, g=FAKE + 4 * SEP, lse=LSE,
             dq=FAKE + 10 * SEP, dk=FAKE + 11 * SEP, dv=FAKE + 12 * SEP, delta=FAKE + 13 * SEP)
    a.update(kw)
    return lib.hv_joint_attention_varlen_bwd(a["q"], a["k"], a["v"], a["o"], a["g"], a["lse"], aq, ak, n,
                                             a["dq"], a["dk"], a["dv"], a["delta"], ctypes.byref(lay),
                                             0.0, None)


@pytest.mark.parametrize("kwargs,expect", [
    (dict(q=0), E), (dict(dk=0), E), (dict(lse=0), E), (dict(delta=LSE + 128), E),
    (dict(n=0), E), (dict(cq=(0, 100, 301)), E), (dict(cq=(0, 120, 100)), E),
    (dict(cq=(0, 100, 300), ck=(0, 100, 100)), E),
    (dict(lay=layout(batch=2, sb=300 * 3072)), E),
    (dict(dv=FAKE + 2 * SEP + 64), E),
    (dict(lay=layout(heads=12)), U),
])
def test_varlen_bwd_validation(kwargs, expect):
    assert varlen_bwd(**kwargs) == expect


def test_varlen_bwd_empty_segments_launch_nothing():
    assert varlen_bwd(cq=(0, 0, 0), ck=(0, 0, 0)) == hv.HV_OK


# ------------------------------------------------- packed-V workspace (forward)
WS = FAKE + 20 * SEP
TILE_BYTES = 24 * 64 * 128 * 2      # one 64-key tile of packed V for all heads
COUNTER = 256                        # the attention's work counter after the packed V


@pytest.mark.parametrize("n_keys,n_seg,tiles", [
    (0, 0, 0), (1, 1, 1), (64, 1, 1), (65, 1, 2), (300, 1, 5), (119056, 1, 1861),
    (2 * 300, 2, 11), (100, 3, 4), (-1, 1, 0), (5, -1, 0),   # floor((n + 63 s) / 64) tiles
])
def test_workspace_bytes(n_keys, n_seg, tiles):
    assert hv.hv_attention_workspace_bytes(n_keys, n_seg) == (tiles * TILE_BYTES + COUNTER if tiles else 0)


def test_workspace_bound_covers_every_split():
    # sum over segments of ceil(k / 64) never exceeds the bound for their total
    import random
    r = random.Random(5)
    for _ in range(2000):
        ks = [r.randint(0, 300) for _ in range(r.randint(1, 64))]
        tiles = sum((k + 63) // 64 for k in ks)
        need = tiles * TILE_BYTES + COUNTER if tiles else 0
        assert need <= hv.hv_attention_workspace_bytes(sum(ks), len(ks))


# default attn(): one segment of 40 + 10 keys = 1 tile; attn_lse(): 300 keys = 5
# tiles; varlen(): segments of 100 and 200 keys = 2 + 4 tiles
@pytest.mark.parametrize("call,need", [(attn, TILE_BYTES + COUNTER), (attn_lse, 5 * TILE_BYTES + COUNTER),
                                       (varlen, 6 * TILE_BYTES + COUNTER)])
def test_workspace_validation(call, need):
    assert call(ws=WS, ws_bytes=need - 1) == E                  # too small
    assert call(ws=WS, ws_bytes=0) == E
    assert call(ws=WS + 8, ws_bytes=need + 64) == E             # not 16-byte aligned
    assert call(ws=WS, ws_bytes=-1) == E
    assert call(ws=None, ws_bytes=-1) == E
    assert call(ws=FAKE + 64, ws_bytes=need) == E               # inside q
    assert call(ws=FAKE + SEP - 1024, ws_bytes=need) == E       # runs into k
    assert call(ws=FAKE + 2 * SEP + 4096, ws_bytes=need) == E   # inside v
    assert call(ws=FAKE + 3 * SEP, ws_bytes=need) == E          # is out


def test_workspace_must_not_meet_lse():
    need = 6 * TILE_BYTES + COUNTER
    assert attn_lse(ws=LSE - 128, ws_bytes=5 * TILE_BYTES + COUNTER) == E
    assert varlen(ws=LSE + 256, ws_bytes=need) == E

