"""rope_joint_attention_amd: Python binding of libhvattn (MI355X / gfx950).

A thin ctypes layer over the C ABI in include/hvattn.h.  The functions keep
the C names and only marshal arguments: torch tensors become device pointers
and strides, the current torch stream becomes the HIP stream.  Every step of
the computation runs in the HIP kernels of libhvattn.so; if the library is
not built, every call raises (there is no fallback).

    hv_token_grid(frames, height, width) -> HvGrid
    hv_rope3d_apply(q, k, grid, theta)          # in place on video rows
    hv_qk_norm_rope3d_apply(q, k, grid, theta, gamma_q, gamma_k,
                            gamma_q_text=None, gamma_k_text=None, eps=1e-6)
    hv_attention_workspace_bytes(n_keys, n_segments) -> int
    hv_joint_attention_fwd(q, k, v, text_valid_len, n_video, out=None,
                           softmax_scale=None, workspace=None, pack_v=True) -> out
    hv_attention_fwd_lse(q, k, v, kv_valid_len=None, ...) -> (out, lse)
    hv_attention_merge(outs, lses, ...) -> (out, lse)
    hv_joint_attention_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k=None,
                                  ...) -> (out, lse)
    hv_joint_attention_bwd(q, k, v, out, dout, lse, text_valid_len, n_video,
                           ...) -> (dq, dk, dv)
    hv_joint_attention_bwd_noalloc(q, k, v, out, dout, lse, text_valid_len,
                                   n_video, dq, dk, dv) -> (dq, dk, dv)
    hv_joint_attention_varlen_bwd(q, k, v, out, dout, lse, cu_seqlens_q,
                                  cu_seqlens_k=None, ...) -> (dq, dk, dv)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "HV_HEADS", "HV_HEAD_DIM", "HV_MAX_BATCH", "HvError", "HvGrid",
    "hv_token_grid", "hv_rope3d_apply", "hv_qk_norm_rope3d_apply", "hv_attention_workspace_bytes",
    "hv_joint_attention_fwd",
    "hv_attention_fwd_lse", "hv_attention_merge", "hv_joint_attention_varlen_fwd",
    "hv_joint_attention_bwd", "hv_joint_attention_bwd_noalloc", "hv_joint_attention_varlen_bwd",
    "hv_status_string", "library_path", "load_library",
]

HV_HEADS = 24
HV_HEAD_DIM = 128
HV_MAX_BATCH = 64
HV_MAX_SEGMENTS = 64
HV_MAX_MERGE_PARTS = 16
HV_NOALLOC_BWD_SCRATCH_BYTES = (32 << 20) + 256
HV_OK, HV_ERR_INVALID_ARG, HV_ERR_UNSUPPORTED, HV_ERR_HIP = 0, -1, -2, -3

_PKG = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    """Path of the library to load: $HVATTN_LIBRARY when set (another build
    of the same sources, e.g. the host-sanitizer build), else the in-tree
    lib/libhvattn.so."""
    return os.environ.get("HVATTN_LIBRARY") or os.path.join(_PKG, "lib", "libhvattn.so")


class HvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {hv_status_string(status)} (status {status})")


class _Grid(ctypes.Structure):
    _fields_ = [("frames", ctypes.c_int32), ("height", ctypes.c_int32), ("width", ctypes.c_int32),
                ("t_lat", ctypes.c_int32), ("h_lat", ctypes.c_int32), ("w_lat", ctypes.c_int32),
                ("gt", ctypes.c_int32), ("gh", ctypes.c_int32), ("gw", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("n_video", ctypes.c_int64)]


class _Layout(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("stride_b", ctypes.c_int64), ("stride_l", ctypes.c_int64)]


class HvGrid:
    """Result of hv_token_grid (mirrors struct hv_grid)."""

    __slots__ = ("frames", "height", "width", "t_lat", "h_lat", "w_lat", "gt", "gh", "gw", "n_video")

    def __init__(self, g: _Grid):
        for name in self.__slots__:
            setattr(self, name, int(getattr(g, name)))

    def _c(self) -> _Grid:
        g = _Grid()
        for name in self.__slots__:
            setattr(g, name, getattr(self, name))
        return g

    def __repr__(self):
        return ("HvGrid(" + ", ".join(f"{n}={getattr(self, n)}" for n in self.__slots__) + ")")


_lib = None


def load_library():
    """Load libhvattn.so from the package directory (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libhvattn.so is not built ({path}); run "
                           f"`python -m rope_joint_attention_amd.build`")
    lib = ctypes.CDLL(path)
    lib.hv_token_grid.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_Grid)]
    lib.hv_token_grid.restype = ctypes.c_int
    lib.hv_rope3d_apply.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_Layout),
                                    ctypes.POINTER(_Grid), ctypes.c_float, ctypes.c_void_p]
    lib.hv_rope3d_apply.restype = ctypes.c_int
    lib.hv_qk_norm_rope3d_apply.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_Layout),
                                            ctypes.POINTER(_Grid), ctypes.c_float,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p]
    lib.hv_qk_norm_rope3d_apply.restype = ctypes.c_int
    lib.hv_joint_attention_fwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p,
                                           ctypes.POINTER(_Layout), ctypes.c_int64, ctypes.c_float,
                                           ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.hv_joint_attention_fwd.restype = ctypes.c_int
    lib.hv_attention_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32]
    lib.hv_attention_workspace_bytes.restype = ctypes.c_int64
    lib.hv_attention_fwd_lse.argtypes = [ctypes.c_void_p, ctypes.POINTER(_Layout), ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.POINTER(_Layout),
                                         ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_void_p]
    lib.hv_attention_fwd_lse.restype = ctypes.c_int
    lib.hv_attention_merge.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.POINTER(_Layout), ctypes.c_void_p]
    lib.hv_attention_merge.restype = ctypes.c_int
    lib.hv_joint_attention_varlen_fwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.POINTER(ctypes.c_int32),
                                                  ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                                  ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.POINTER(_Layout), ctypes.c_float,
                                                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.hv_joint_attention_varlen_fwd.restype = ctypes.c_int
    lib.hv_joint_attention_bwd.argtypes = [ctypes.c_void_p] * 6 + [
        ctypes.POINTER(ctypes.c_int32), ctypes.c_int64] + [ctypes.c_void_p] * 4 + [
        ctypes.POINTER(_Layout), ctypes.c_float, ctypes.c_void_p]
    lib.hv_joint_attention_bwd.restype = ctypes.c_int
    lib.hv_joint_attention_bwd_noalloc.argtypes = [ctypes.c_void_p] * 6 + [
        ctypes.POINTER(ctypes.c_int32), ctypes.c_int64] + [ctypes.c_void_p] * 3 + [
        ctypes.POINTER(_Layout), ctypes.c_float, ctypes.c_void_p]
    lib.hv_joint_attention_bwd_noalloc.restype = ctypes.c_int
    lib.hv_joint_attention_varlen_bwd.argtypes = [ctypes.c_void_p] * 6 + [
        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), ctypes.c_int32] + [
        ctypes.c_void_p] * 4 + [ctypes.POINTER(_Layout), ctypes.c_float, ctypes.c_void_p]
    lib.hv_joint_attention_varlen_bwd.restype = ctypes.c_int
    lib.hv_status_string.argtypes = [ctypes.c_int]
    lib.hv_status_string.restype = ctypes.c_char_p
    lib.hv_version.argtypes = []
    lib.hv_version.restype = ctypes.c_int
    _lib = lib
    return lib


def hv_status_string(status: int) -> str:
    return load_library().hv_status_string(int(status)).decode()


def hv_token_grid(frames: int, height: int, width: int) -> HvGrid:
    g = _Grid()
    st = load_library().hv_token_grid(int(frames), int(height), int(width), ctypes.byref(g))
    if st != HV_OK:
        raise HvError(st, f"hv_token_grid({frames}, {height}, {width})")
    return HvGrid(g)


def _layout_of(t, what: str) -> _Layout:
    import torch

    if t.dtype != torch.bfloat16:
        raise TypeError(f"{what} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{what} must be a GPU tensor")
    if t.dim() != 4 or t.shape[2] != HV_HEADS or t.shape[3] != HV_HEAD_DIM:
        raise ValueError(f"{what} must be [batch, seq, {HV_HEADS}, {HV_HEAD_DIM}], got {tuple(t.shape)}")
    if t.stride(3) != 1 or t.stride(2) != HV_HEAD_DIM:
        raise ValueError(f"{what} needs contiguous heads x channels, strides {t.stride()}")
    lay = _Layout()
    lay.batch, lay.seq_len = t.shape[0], t.shape[1]
    lay.heads, lay.head_dim = HV_HEADS, HV_HEAD_DIM
    lay.stride_b, lay.stride_l = t.stride(0), t.stride(1)
    return lay


def _same_layout(a: _Layout, b: _Layout) -> bool:
    return all(getattr(a, f) == getattr(b, f) for f, _ in _Layout._fields_)


def _stream_of(t):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def hv_rope3d_apply(q, k, grid: HvGrid, theta: float = 10000.0) -> None:
    """Rotate the video rows of q and k in place (see hvattn.h)."""
    lay = _layout_of(q, "q")
    if not _same_layout(lay, _layout_of(k, "k")):
        raise ValueError("q and k must share shape and strides")
    g = grid._c()
    st = load_library().hv_rope3d_apply(q.data_ptr(), k.data_ptr(), ctypes.byref(lay),
                                        ctypes.byref(g), float(theta), _stream_of(q))
    if st != HV_OK:
        raise HvError(st, "hv_rope3d_apply")


def _weight_ptr(g, what: str, device) -> Optional[int]:
    import torch

    if g is None:
        return None
    if g.dtype != torch.bfloat16 or g.device != device:
        raise TypeError(f"{what} must be a bfloat16 tensor on {device}")
    if g.dim() != 1 or g.shape[0] != HV_HEAD_DIM or g.stride(0) != 1:
        raise ValueError(f"{what} must be a contiguous [{HV_HEAD_DIM}] vector, got {tuple(g.shape)}")
    return g.data_ptr()


def hv_qk_norm_rope3d_apply(q, k, grid: HvGrid, theta: float, gamma_q, gamma_k,
                            gamma_q_text=None, gamma_k_text=None, eps: float = 1e-6) -> None:
    """Per-head RMSNorm of every row of q and k, then 3D RoPE of the video rows,
    in place (see hvattn.h).  gamma_* are bfloat16 [128] device vectors; the text
    weights default to the video ones."""
    lay = _layout_of(q, "q")
    if not _same_layout(lay, _layout_of(k, "k")):
        raise ValueError("q and k must share shape and strides")
    g = grid._c()
    ptrs = [_weight_ptr(w, n, q.device) for w, n in ((gamma_q, "gamma_q"), (gamma_k, "gamma_k"),
                                                     (gamma_q_text, "gamma_q_text"),
                                                     (gamma_k_text, "gamma_k_text"))]
    st = load_library().hv_qk_norm_rope3d_apply(q.data_ptr(), k.data_ptr(), ctypes.byref(lay),
                                                ctypes.byref(g), float(theta), *ptrs, float(eps),
                                                _stream_of(q))
    if st != HV_OK:
        raise HvError(st, "hv_qk_norm_rope3d_apply")


def hv_attention_workspace_bytes(n_keys: int, n_segments: int) -> int:
    """Upper bound of the packed-V workspace of a forward call (see hvattn.h)."""
    return int(load_library().hv_attention_workspace_bytes(int(n_keys), int(n_segments)))


def _workspace(workspace, pack_v: bool, nbytes: int, device):
    """(pointer, bytes) of the packed-V workspace: the given tensor, a fresh
    one of nbytes from torch's allocator, or (None, 0) for the in-place path."""
    import torch

    if workspace is not None:
        if not workspace.is_cuda or workspace.device != device or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {device}")
        return workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if not pack_v:
        return None, 0
    # torch's allocator hands the block to later allocations on the same
    # stream only, which run after this call's kernels: freeing it when this
    # function returns is safe
    ws = torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)
    return ws.data_ptr(), nbytes


def hv_joint_attention_fwd(q, k, v, text_valid_len: Optional[Sequence[int]], n_video: int,
                           out=None, softmax_scale: Optional[float] = None, workspace=None,
                           pack_v: bool = True):
    """Joint [video; text] attention forward (see hvattn.h); returns out.
    workspace: device tensor for the packed V (hv_attention_workspace_bytes
    (batch * seq_len, batch) bytes); by default one is taken from torch's
    allocator; pack_v=False (and no workspace) reads V in place."""
    import torch

    lay = _layout_of(q, "q")
    for t, name in ((k, "k"), (v, "v")):
        if not _same_layout(lay, _layout_of(t, name)):
            raise ValueError(f"q and {name} must share shape and strides")
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    elif not _same_layout(lay, _layout_of(out, "out")):
        raise ValueError("out must share shape and strides with q")
    valid_arr = None
    if text_valid_len is not None:
        vals = [int(x) for x in text_valid_len]
        if len(vals) != q.shape[0]:
            raise ValueError("text_valid_len needs one entry per batch element")
        valid_arr = (ctypes.c_int32 * max(1, len(vals)))(*vals)
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    wptr, wbytes = _workspace(workspace, pack_v,
                              hv_attention_workspace_bytes(q.shape[0] * q.shape[1], q.shape[0]),
                              q.device)
    st = load_library().hv_joint_attention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), valid_arr,
                                               out.data_ptr(), ctypes.byref(lay), int(n_video),
                                               scale, wptr, wbytes, _stream_of(q))
    if st != HV_OK:
        raise HvError(st, "hv_joint_attention_fwd")
    return out


def _lse_buffer(lse, shape, device, what: str):
    import torch

    if lse is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    if lse.dtype != torch.float32 or lse.device != device or tuple(lse.shape) != tuple(shape) \
            or not lse.is_contiguous():
        raise ValueError(f"{what} must be a contiguous float32 tensor of shape {tuple(shape)}")
    return lse


BWD_COUNTER_FLOATS = 64   # the 256 bytes of work counters after D in the backward's workspace


def _delta_workspace(delta, n_rows: int, device):
    """The backward's delta workspace: n_rows * 24 floats of -D, as many of
    -lse/scale, then the counters.  A given tensor must be a contiguous float32
    tensor with at least that many elements."""
    import torch

    need = 2 * n_rows * HV_HEADS + BWD_COUNTER_FLOATS
    if delta is None:
        return torch.empty(need, dtype=torch.float32, device=device)
    if delta.dtype != torch.float32 or delta.device != device or not delta.is_contiguous() \
            or delta.numel() < need:
        raise ValueError(f"delta must be a contiguous float32 tensor of at least {need} elements "
                         f"(2 x 24 per row, then {BWD_COUNTER_FLOATS} for the work counters)")
    return delta


def hv_attention_fwd_lse(q, k, v, kv_valid_len: Optional[Sequence[int]] = None, out=None,
                         lse=None, want_lse: bool = True, softmax_scale: Optional[float] = None,
                         workspace=None, pack_v: bool = True):
    """Attention of q's rows against a separate K/V block, with the natural-log
    log-sum-exp of every row (see hvattn.h).  q: [B, Lq, 24, 128], k and v:
    [B, Lk, 24, 128] (sharing shape and strides).  Returns (out, lse) with lse
    float32 [B, 24, Lq] (None when want_lse is False and no lse is given).
    workspace / pack_v as in hv_joint_attention_fwd (n_keys = B * Lk)."""
    import torch

    qlay = _layout_of(q, "q")
    kvlay = _layout_of(k, "k")
    if not _same_layout(kvlay, _layout_of(v, "v")):
        raise ValueError("k and v must share shape and strides")
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    elif not _same_layout(qlay, _layout_of(out, "out")):
        raise ValueError("out must share shape and strides with q")
    if lse is not None or want_lse:
        lse = _lse_buffer(lse, (q.shape[0], HV_HEADS, q.shape[1]), q.device, "lse")
    valid_arr = None
    if kv_valid_len is not None:
        vals = [int(x) for x in kv_valid_len]
        if len(vals) != q.shape[0]:
            raise ValueError("kv_valid_len needs one entry per batch element")
        valid_arr = (ctypes.c_int32 * max(1, len(vals)))(*vals)
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    wptr, wbytes = _workspace(workspace, pack_v,
                              hv_attention_workspace_bytes(k.shape[0] * k.shape[1], k.shape[0]),
                              q.device)
    st = load_library().hv_attention_fwd_lse(q.data_ptr(), ctypes.byref(qlay), k.data_ptr(),
                                             v.data_ptr(), ctypes.byref(kvlay), valid_arr,
                                             out.data_ptr(), None if lse is None else lse.data_ptr(),
                                             scale, wptr, wbytes, _stream_of(q))
    if st != HV_OK:
        raise HvError(st, "hv_attention_fwd_lse")
    return out, lse


def hv_attention_merge(outs, lses, out=None, lse_out=None, want_lse: bool = True):
    """Combine attention results over disjoint key blocks (see hvattn.h).
    outs: list of [B, L, 24, 128] bf16 tensors sharing shape and strides; lses:
    matching float32 [B, 24, L].  Returns (out, lse_out)."""
    import torch

    if len(outs) != len(lses) or not 1 <= len(outs) <= HV_MAX_MERGE_PARTS:
        raise ValueError(f"need 1..{HV_MAX_MERGE_PARTS} (out, lse) pairs")
    lay = _layout_of(outs[0], "outs[0]")
    shape = (outs[0].shape[0], HV_HEADS, outs[0].shape[1])
    for i, (o, l) in enumerate(zip(outs, lses)):
        if not _same_layout(lay, _layout_of(o, f"outs[{i}]")):
            raise ValueError("all partial outputs must share shape and strides")
        _lse_buffer(l, shape, outs[0].device, f"lses[{i}]")
    if out is None:
        out = torch.empty_strided(outs[0].shape, outs[0].stride(), dtype=outs[0].dtype,
                                  device=outs[0].device)
    elif not _same_layout(lay, _layout_of(out, "out")):
        raise ValueError("out must share shape and strides with the partial outputs")
    if lse_out is not None or want_lse:
        lse_out = _lse_buffer(lse_out, shape, outs[0].device, "lse_out")
    n = len(outs)
    optrs = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    lptrs = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lses])
    st = load_library().hv_attention_merge(optrs, lptrs, n, out.data_ptr(),
                                           None if lse_out is None else lse_out.data_ptr(),
                                           ctypes.byref(lay), _stream_of(out))
    if st != HV_OK:
        raise HvError(st, "hv_attention_merge")
    return out, lse_out


def hv_joint_attention_varlen_fwd(q, k, v, cu_seqlens_q: Sequence[int],
                                  cu_seqlens_k: Optional[Sequence[int]] = None, out=None, lse=None,
                                  want_lse: bool = False, softmax_scale: Optional[float] = None,
                                  workspace=None, pack_v: bool = True):
    """Attention over packed segments (see hvattn.h).  q, k, v: [T, 24, 128]
    packed rows sharing shape and strides; cu_seqlens_*: segment offsets
    (cu_seqlens_k defaults to cu_seqlens_q).  Returns (out, lse) with lse
    float32 [24, T] or None.  workspace / pack_v as in hv_joint_attention_fwd
    (n_keys = T)."""
    import torch

    def as4(t, name):
        if t.dim() != 3:
            raise ValueError(f"{name} must be [T, {HV_HEADS}, {HV_HEAD_DIM}]")
        return t.unsqueeze(0)

    q4, k4, v4 = as4(q, "q"), as4(k, "k"), as4(v, "v")
    lay = _layout_of(q4, "q")
    for t, name in ((k4, "k"), (v4, "v")):
        if not _same_layout(lay, _layout_of(t, name)):
            raise ValueError(f"q and {name} must share shape and strides")
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    elif not _same_layout(lay, _layout_of(as4(out, "out"), "out")):
        raise ValueError("out must share shape and strides with q")
    if lse is not None or want_lse:
        lse = _lse_buffer(lse, (HV_HEADS, q.shape[0]), q.device, "lse")
    cq = [int(x) for x in cu_seqlens_q]
    ck = cq if cu_seqlens_k is None else [int(x) for x in cu_seqlens_k]
    if len(cq) != len(ck) or len(cq) < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need n_segments + 1 entries each")
    aq = (ctypes.c_int32 * len(cq))(*cq)
    ak = (ctypes.c_int32 * len(ck))(*ck)
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    wptr, wbytes = _workspace(workspace, pack_v,
                              hv_attention_workspace_bytes(q.shape[0], len(cq) - 1), q.device)
    st = load_library().hv_joint_attention_varlen_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), aq, ak,
                                                      len(cq) - 1, out.data_ptr(),
                                                      None if lse is None else lse.data_ptr(),
                                                      ctypes.byref(lay), scale, wptr, wbytes,
                                                      _stream_of(q))
    if st != HV_OK:
        raise HvError(st, "hv_joint_attention_varlen_fwd")
    return out, lse


def hv_joint_attention_bwd(q, k, v, out, dout, lse, text_valid_len: Optional[Sequence[int]],
                           n_video: int, dq=None, dk=None, dv=None, delta=None,
                           softmax_scale: Optional[float] = None):
    """Gradients of hv_joint_attention_fwd (see hvattn.h).  q, k, v, out, dout
    share shape [B, L, 24, 128] and strides; lse is the forward's float32
    [B, 24, L] log-sum-exp (hv_attention_fwd_lse).  Returns (dq, dk, dv)."""
    import torch

    lay = _layout_of(q, "q")
    for t, name in ((k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        if not _same_layout(lay, _layout_of(t, name)):
            raise ValueError(f"q and {name} must share shape and strides")
    shape = (q.shape[0], HV_HEADS, q.shape[1])
    _lse_buffer(lse, shape, q.device, "lse")
    delta = _delta_workspace(delta, q.shape[0] * q.shape[1], q.device)
    grads = []
    for g, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if g is None:
            g = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
        elif not _same_layout(lay, _layout_of(g, name)):
            raise ValueError(f"{name} must share shape and strides with q")
        grads.append(g)
    valid_arr = None
    if text_valid_len is not None:
        vals = [int(x) for x in text_valid_len]
        if len(vals) != q.shape[0]:
            raise ValueError("text_valid_len needs one entry per batch element")
        valid_arr = (ctypes.c_int32 * max(1, len(vals)))(*vals)
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    st = load_library().hv_joint_attention_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                               out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                                               valid_arr, int(n_video), grads[0].data_ptr(),
                                               grads[1].data_ptr(), grads[2].data_ptr(),
                                               delta.data_ptr(), ctypes.byref(lay), scale,
                                               _stream_of(q))
    if st != HV_OK:
        raise HvError(st, "hv_joint_attention_bwd")
    return tuple(grads)


def hv_joint_attention_bwd_noalloc(q, k, v, out, dout, lse, text_valid_len: Optional[Sequence[int]],
                                   n_video: int, dq, dk, dv, softmax_scale: Optional[float] = None):
    """hv_joint_attention_bwd with the library's static device scratch in place
    of the delta workspace (see hvattn.h): for callers that cannot allocate.
    dq, dk, dv are required (this wrapper allocates nothing either).
    Returns (dq, dk, dv)."""
    lay = _layout_of(q, "q")
    for t, name in ((k, "k"), (v, "v"), (out, "out"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
                    (dv, "dv")):
        if t is None:
            raise ValueError(f"{name} is required")
        if not _same_layout(lay, _layout_of(t, name)):
            raise ValueError(f"q and {name} must share shape and strides")
    if lse is None:
        raise ValueError("lse (the forward's log-sum-exp) is required")
    _lse_buffer(lse, (q.shape[0], HV_HEADS, q.shape[1]), q.device, "lse")
    valid_arr = None
    if text_valid_len is not None:
        vals = [int(x) for x in text_valid_len]
        if len(vals) != q.shape[0]:
            raise ValueError("text_valid_len needs one entry per batch element")
        valid_arr = (ctypes.c_int32 * max(1, len(vals)))(*vals)
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    st = load_library().hv_joint_attention_bwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
        valid_arr, int(n_video), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ctypes.byref(lay),
        scale, _stream_of(q))
    if st != HV_OK:
        raise HvError(st, "hv_joint_attention_bwd_noalloc")
    return dq, dk, dv


def hv_joint_attention_varlen_bwd(q, k, v, out, dout, lse, cu_seqlens_q: Sequence[int],
                                  cu_seqlens_k: Optional[Sequence[int]] = None, dq=None, dk=None,
                                  dv=None, delta=None, softmax_scale: Optional[float] = None):
    """Gradients of hv_joint_attention_varlen_fwd (see hvattn.h).  q, k, v, out,
    dout: [T, 24, 128] packed rows sharing shape and strides; lse: the forward's
    float32 [24, T].  Returns (dq, dk, dv)."""
    import torch

    def as4(t, name):
        if t.dim() != 3:
            raise ValueError(f"{name} must be [T, {HV_HEADS}, {HV_HEAD_DIM}]")
        return t.unsqueeze(0)

    lay = _layout_of(as4(q, "q"), "q")
    for t, name in ((k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        if not _same_layout(lay, _layout_of(as4(t, name), name)):
            raise ValueError(f"q and {name} must share shape and strides")
    shape = (HV_HEADS, q.shape[0])
    _lse_buffer(lse, shape, q.device, "lse")
    delta = _delta_workspace(delta, q.shape[0], q.device)
    grads = []
    for g, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if g is None:
            g = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
        elif not _same_layout(lay, _layout_of(as4(g, name), name)):
            raise ValueError(f"{name} must share shape and strides with q")
        grads.append(g)
    cq = [int(x) for x in cu_seqlens_q]
    ck = cq if cu_seqlens_k is None else [int(x) for x in cu_seqlens_k]
    if len(cq) != len(ck) or len(cq) < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k need n_segments + 1 entries each")
    aq = (ctypes.c_int32 * len(cq))(*cq)
    ak = (ctypes.c_int32 * len(ck))(*ck)
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    st = load_library().hv_joint_attention_varlen_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                      out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                                                      aq, ak, len(cq) - 1, grads[0].data_ptr(),
                                                      grads[1].data_ptr(), grads[2].data_ptr(),
                                                      delta.data_ptr(), ctypes.byref(lay), scale,
                                                      _stream_of(q))
    if st != HV_OK:
        raise HvError(st, "hv_joint_attention_varlen_bwd")
    return tuple(grads)
