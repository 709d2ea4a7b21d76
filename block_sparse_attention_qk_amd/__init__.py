"""Block-sparse video self-attention on MI355X: thin Python binding.

The functions here carry the same names as the C ABI in ``include/sva.h``
and only marshal arguments: torch tensors are checked (dtype, device,
shape, contiguity, alignment) and passed as raw device pointers together
with the current HIP stream.  Every step runs in the HIP kernels of
``libsva.so``; there is no fallback path.  The library is loaded on first
use and a missing or unloadable library raises ``RuntimeError``.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsva.so")
# the same library built with device-side index checks (-DSVA_DEBUG); load it
# by pointing LIB_PATH here before the first call
DEBUG_LIB_PATH = os.path.join(_HERE, "libsva_debug.so")

SVA_OK = 0
SVA_ERR_INVALID_ARG = -1
SVA_ERR_UNSUPPORTED = -2
SVA_ERR_WORKSPACE = -3
SVA_ERR_HIP = -4

SVA_DENSE = 1
SVA_KEEP_SAME_FRAME = 2
SVA_COMPENSATE = 4

SVA_LAYOUT_TILE = 0
SVA_LAYOUT_RASTER = 1

SVA_SCORER_MEAN = 0
SVA_SCORER_SUBBLOCK = 1

SVA_FORWARD = 0
SVA_INVERSE = 1
SVA_FORWARD_VT = 2
SVA_FORWARD_KT = 3
SVA_ROWS_TO_VT = 4
SVA_ROWS_TO_KT = 5

EXPORTED = (
    "sva_plan_desc_init", "sva_plan_query", "sva_plan_host_tables",
    "sva_plan_create", "sva_plan_create_ex", "sva_plan_get_info", "sva_destroy",
    "sva_qk_norm_rope", "sva_reorder", "sva_select_blocks", "sva_attention",
    "sva_block_means", "sva_attention_compensated", "sva_qk_norm_rope_tiled",
    "sva_attention_ex", "sva_attention_ws", "sva_select_blocks_noalloc", "sva_stream_copy",
    "sva_forward", "sva_debug_flags", "sva_debug_selftest", "sva_status_string", "sva_last_error",
)

SVA_DEBUG_TOKEN = 1
SVA_DEBUG_LIST = 2
SVA_DEBUG_ROW = 4
SVA_DEBUG_SELF = 8

SVA_FORWARD_MARKS = 6


class sva_step_buffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q", "k", "v", "wq", "wk", "q_r", "k_t", "v_t", "select_ws")] + [
        ("select_ws_bytes", ctypes.c_size_t), ("col", ctypes.c_void_p),
        ("km_t", ctypes.c_void_p), ("vm_t", ctypes.c_void_p), ("attn_ws", ctypes.c_void_p),
        ("attn_ws_bytes", ctypes.c_size_t), ("o", ctypes.c_void_p)]


class sva_plan_desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("H", ctypes.c_int),
        ("T", ctypes.c_int), ("Hh", ctypes.c_int), ("W", ctypes.c_int),
        ("d", ctypes.c_int), ("block", ctypes.c_int),
        ("sparsity", ctypes.c_double), ("flags", ctypes.c_uint),
        ("tile_t", ctypes.c_int), ("tile_h", ctypes.c_int), ("tile_w", ctypes.c_int),
        ("n_extra", ctypes.c_int),
        ("rope_theta", ctypes.c_double),
        ("rope_split", ctypes.c_int * 3),
        ("eps", ctypes.c_double),
        ("scorer", ctypes.c_int), ("subblocks", ctypes.c_int),
        ("budget_multiple", ctypes.c_int),
    ]


class sva_plan_info(ctypes.Structure):
    _fields_ = [
        ("n_video", ctypes.c_int64), ("N", ctypes.c_int64),
        ("n_video_pad", ctypes.c_int64), ("Np", ctypes.c_int64),
        ("nB", ctypes.c_int32), ("nB_video", ctypes.c_int32),
        ("k", ctypes.c_int32), ("max_row_len", ctypes.c_int32),
        ("nnz_per_head", ctypes.c_int64), ("nnz", ctypes.c_int64),
        ("select_workspace_bytes", ctypes.c_size_t),
        ("dense", ctypes.c_int32),
        ("tile", ctypes.c_int32 * 3),
        ("rope_split", ctypes.c_int32 * 3),
        ("scorer", ctypes.c_int32), ("subblocks", ctypes.c_int32),
        ("budget_multiple", ctypes.c_int32), ("n_mean_groups", ctypes.c_int32),
        ("attention_workspace_bytes", ctypes.c_size_t),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsva.so (once).  Raises RuntimeError when it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_sparse_attention_qk_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, d, u, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_uint, ctypes.c_size_t
    P = ctypes.POINTER
    L.sva_plan_desc_init.argtypes = [P(sva_plan_desc), i, i, i, i, i, i, i, d, u]
    L.sva_plan_query.argtypes = [P(sva_plan_desc), P(sva_plan_info)]
    L.sva_plan_host_tables.argtypes = [P(sva_plan_desc), vp, vp, vp]
    L.sva_plan_create.argtypes = [P(vp), i, i, i, i, i, i, i, d, u]
    L.sva_plan_create_ex.argtypes = [P(vp), P(sva_plan_desc)]
    L.sva_plan_get_info.argtypes = [vp, P(sva_plan_info)]
    L.sva_destroy.argtypes = [vp]
    L.sva_qk_norm_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
    L.sva_reorder.argtypes = [vp, vp, vp, i, vp]
    L.sva_select_blocks.argtypes = [vp, vp, vp, vp, sz, vp, vp]
    L.sva_select_blocks_noalloc.argtypes = [vp, vp, vp, vp, vp]
    L.sva_stream_copy.argtypes = [vp, vp, sz, vp]
    L.sva_attention.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    L.sva_block_means.argtypes = [vp, vp, vp, vp, vp, vp]
    L.sva_attention_compensated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.sva_qk_norm_rope_tiled.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.sva_attention_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, vp]
    L.sva_attention_ws.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, vp, sz, vp]
    L.sva_forward.argtypes = [vp, P(sva_step_buffers), vp, vp]
    L.sva_debug_flags.argtypes = [vp, P(u)]
    L.sva_debug_selftest.argtypes = [vp, vp]
    L.sva_status_string.argtypes = [i]
    L.sva_status_string.restype = ctypes.c_char_p
    L.sva_last_error.argtypes = []
    L.sva_last_error.restype = ctypes.c_char_p
    for name in EXPORTED:
        if name not in ("sva_status_string", "sva_last_error"):
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


class SvaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sva status {status}: {msg}")
        self.status = status


def _check(status: int) -> None:
    if status != SVA_OK:
        raise SvaError(status, lib().sva_last_error().decode())


# --------------------------------------------------------------------------
# host-only calls
# --------------------------------------------------------------------------

def sva_plan_desc_init(B, H, T, Hh, W, d, block, sparsity, flags=0, tile=(0, 0, 0),
                       n_extra=0, rope_theta=0.0, rope_split=(0, 0, 0), eps=0.0,
                       scorer=SVA_SCORER_MEAN, subblocks=0, budget_multiple=0) -> sva_plan_desc:
    desc = sva_plan_desc()
    _check(lib().sva_plan_desc_init(ctypes.byref(desc), B, H, T, Hh, W, d, block,
                                    float(sparsity), flags))
    desc.tile_t, desc.tile_h, desc.tile_w = tile
    desc.n_extra = n_extra
    desc.rope_theta = rope_theta
    desc.rope_split[:] = list(rope_split)
    desc.eps = eps
    desc.scorer = scorer
    desc.subblocks = subblocks
    desc.budget_multiple = budget_multiple
    return desc


def sva_plan_query(desc: sva_plan_desc) -> sva_plan_info:
    info = sva_plan_info()
    _check(lib().sva_plan_query(ctypes.byref(desc), ctypes.byref(info)))
    return info


def sva_plan_host_tables(desc: sva_plan_desc, forced: bool = False):
    """(perm [N] int32, row_ptr [nB+1] int32, forced [nB, nB] uint8 or None)."""
    info = sva_plan_query(desc)
    perm = np.empty(info.N, dtype=np.int32)
    row_ptr = np.empty(info.nB + 1, dtype=np.int32)
    f = np.empty((info.nB, info.nB), dtype=np.uint8) if forced else None
    _check(lib().sva_plan_host_tables(ctypes.byref(desc), perm.ctypes.data,
                                      row_ptr.ctypes.data,
                                      f.ctypes.data if f is not None else None))
    return perm, row_ptr, f


def desc_for(wl) -> sva_plan_desc:
    """Plan description of a workload from ``inputs.WORKLOADS``."""
    return sva_plan_desc_init(wl.B, wl.H, wl.T, wl.Hh, wl.W, wl.d, wl.block, wl.sparsity,
                              wl.flags, tile=wl.tile, n_extra=wl.n_extra,
                              rope_split=getattr(wl, "rope_split", (0, 0, 0)),
                              scorer=getattr(wl, "scorer", SVA_SCORER_MEAN),
                              subblocks=getattr(wl, "subblocks", 0),
                              budget_multiple=getattr(wl, "budget_multiple", 0),
                              rope_theta=getattr(wl, "rope_theta", 0.0),
                              eps=getattr(wl, "eps", 0.0))


# --------------------------------------------------------------------------
# device calls (torch tensors)
# --------------------------------------------------------------------------

def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _tensor(t, shape, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")
    return ctypes.c_void_p(t.data_ptr())


@dataclass
class Plan:
    """A plan on the current device; wraps the C handle."""

    handle: ctypes.c_void_p
    desc: sva_plan_desc
    info: sva_plan_info

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _lib is not None:
            _lib.sva_destroy(h)
            self.handle = None

    # shapes
    @property
    def raster_shape(self):
        d = self.desc
        return (d.B, int(self.info.N), d.H, d.d)

    @property
    def tile_shape(self):
        d = self.desc
        return (d.B, d.H, int(self.info.Np), d.d)

    @property
    def vt_shape(self):
        d = self.desc
        return (d.B, d.H, int(self.info.nB), d.block // 32, 4, d.d, 8)

    @property
    def kt_shape(self):
        d = self.desc
        return (d.B, d.H, int(self.info.nB), d.block // 32, d.d // 16, 64, 8)

    @property
    def km_shape(self):
        d = self.desc
        return (d.B, d.H, int(self.info.n_mean_groups), d.d // 16, 64, 8)

    @property
    def vm_shape(self):
        d = self.desc
        return (d.B, d.H, int(self.info.n_mean_groups), 4, d.d, 8)

    @property
    def compensated(self) -> bool:
        return bool(self.desc.flags & SVA_COMPENSATE) and not self.info.dense

    def host_tables(self, forced=False):
        return sva_plan_host_tables(self.desc, forced)


def sva_plan_create(B, H, T, Hh, W, d, block, sparsity, dense_flag=0) -> Plan:
    h = ctypes.c_void_p()
    _check(lib().sva_plan_create(ctypes.byref(h), B, H, T, Hh, W, d, block, float(sparsity),
                                 dense_flag))
    info = sva_plan_info()
    _check(lib().sva_plan_get_info(h, ctypes.byref(info)))
    # the description with the same defaults (host only), for the shape helpers
    return Plan(h, sva_plan_desc_init(B, H, T, Hh, W, d, block, sparsity, dense_flag), info)


def sva_plan_create_ex(desc: sva_plan_desc) -> Plan:
    h = ctypes.c_void_p()
    _check(lib().sva_plan_create_ex(ctypes.byref(h), ctypes.byref(desc)))
    info = sva_plan_info()
    _check(lib().sva_plan_get_info(h, ctypes.byref(info)))
    return Plan(h, desc, info)


def sva_plan_get_info(plan: Plan) -> sva_plan_info:
    info = sva_plan_info()
    _check(lib().sva_plan_get_info(plan.handle, ctypes.byref(info)))
    return info


def sva_destroy(plan: Plan) -> None:
    if plan.handle is not None and plan.handle.value:
        _check(lib().sva_destroy(plan.handle))
    plan.handle = None


def sva_qk_norm_rope(plan: Plan, q, k, wq, wk, q_out, k_out, stream=None) -> None:
    import torch
    shp = plan.raster_shape
    wshape = (plan.desc.H, plan.desc.d)
    args = [
        _tensor(q, shp, torch.bfloat16, "q"), _tensor(k, shp, torch.bfloat16, "k"),
        _tensor(wq, wshape, torch.float32, "wq") if wq is not None else None,
        _tensor(wk, wshape, torch.float32, "wk") if wk is not None else None,
        _tensor(q_out, shp, torch.bfloat16, "q_out"), _tensor(k_out, shp, torch.bfloat16, "k_out"),
    ]
    _check(lib().sva_qk_norm_rope(plan.handle, *args, _stream(stream)))


def _workspace(workspace):
    if workspace is None:
        return None, 0
    if not (workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def sva_qk_norm_rope_tiled(plan: Plan, q, k, wq, wk, q_r, k_t, workspace=None,
                           stream=None) -> None:
    """Tiled prologue; with ``workspace`` (the select workspace) it also
    writes the block means sva_select_blocks(q_r=None, k_t=None) ranks."""
    import torch
    shp = plan.raster_shape
    wshape = (plan.desc.H, plan.desc.d)
    args = [
        _tensor(q, shp, torch.bfloat16, "q"), _tensor(k, shp, torch.bfloat16, "k"),
        _tensor(wq, wshape, torch.float32, "wq") if wq is not None else None,
        _tensor(wk, wshape, torch.float32, "wk") if wk is not None else None,
        _tensor(q_r, plan.tile_shape, torch.bfloat16, "q_r"),
        _tensor(k_t, plan.kt_shape, torch.bfloat16, "k_t"),
    ]
    ws, ws_bytes = _workspace(workspace)
    _check(lib().sva_qk_norm_rope_tiled(plan.handle, *args, ws, ws_bytes, _stream(stream)))


def sva_reorder(plan: Plan, inp, out, direction, stream=None) -> None:
    import torch
    if direction == SVA_FORWARD:
        si, so = plan.raster_shape, plan.tile_shape
    elif direction == SVA_INVERSE:
        si, so = plan.tile_shape, plan.raster_shape
    elif direction == SVA_FORWARD_VT:
        si, so = plan.raster_shape, plan.vt_shape
    elif direction == SVA_FORWARD_KT:
        si, so = plan.raster_shape, plan.kt_shape
    elif direction == SVA_ROWS_TO_VT:
        si, so = plan.tile_shape, plan.vt_shape
    elif direction == SVA_ROWS_TO_KT:
        si, so = plan.tile_shape, plan.kt_shape
    else:
        raise ValueError("unknown direction")
    _check(lib().sva_reorder(plan.handle, _tensor(inp, si, torch.bfloat16, "in"),
                             _tensor(out, so, torch.bfloat16, "out"), direction, _stream(stream)))


def sva_select_blocks(plan: Plan, q_r, k_t, workspace, col, stream=None) -> None:
    """q_r = k_t = None: rank the means the tiled prologue left in
    ``workspace``."""
    import torch
    if plan.info.dense:
        return
    ts = plan.tile_shape
    if workspace is None:
        raise ValueError("workspace is required")
    ws, ws_bytes = _workspace(workspace)
    _check(lib().sva_select_blocks(
        plan.handle, _tensor(q_r, ts, torch.bfloat16, "q_r") if q_r is not None else None,
        _tensor(k_t, plan.kt_shape, torch.bfloat16, "k_t") if k_t is not None else None,
        ws, ws_bytes, _tensor(col, (int(plan.info.nnz),), torch.int32, "col"), _stream(stream)))


def sva_select_blocks_noalloc(plan: Plan, q_r, k_t, col, stream=None) -> None:
    """sva_select_blocks with the library's fixed device scratch in place of
    a workspace (no allocation; calls that overlap on one GPU race)."""
    import torch
    if plan.info.dense:
        return
    _check(lib().sva_select_blocks_noalloc(
        plan.handle, _tensor(q_r, plan.tile_shape, torch.bfloat16, "q_r"),
        _tensor(k_t, plan.kt_shape, torch.bfloat16, "k_t"),
        _tensor(col, (int(plan.info.nnz),), torch.int32, "col"), _stream(stream)))


def sva_debug_flags(plan: Plan) -> int:
    """Waits for the device, returns the plan's debug word (SVA_DEBUG_*
    bits) and clears it.  Raises SvaError (SVA_ERR_UNSUPPORTED) with a
    release library."""
    flags = ctypes.c_uint(0)
    _check(lib().sva_debug_flags(plan.handle, ctypes.byref(flags)))
    return int(flags.value)


def sva_debug_selftest(plan: Plan, stream=None) -> None:
    """Enqueues the kernel whose check fails on purpose (sets SVA_DEBUG_SELF
    in a debug library)."""
    _check(lib().sva_debug_selftest(plan.handle, _stream(stream)))


def sva_stream_copy(dst, src, stream=None) -> None:
    """Plain streaming copy of src into dst (same size, device tensors):
    the measurement reference for the HBM-bound kernels."""
    for t, n in ((dst, "dst"), (src, "src")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst and src differ in size")
    _check(lib().sva_stream_copy(ctypes.c_void_p(dst.data_ptr()),
                                 ctypes.c_void_p(src.data_ptr()), nbytes, _stream(stream)))


def sva_attention(plan: Plan, q_r, k_t, v_t, col, o_r, stream=None) -> None:
    import torch
    ts = plan.tile_shape
    c = None
    if col is not None:
        c = _tensor(col, (int(plan.info.nnz),), torch.int32, "col")
    elif not plan.info.dense:
        raise ValueError("col is required for a sparse plan")
    _check(lib().sva_attention(plan.handle, _tensor(q_r, ts, torch.bfloat16, "q_r"),
                               _tensor(k_t, plan.kt_shape, torch.bfloat16, "k_t"),
                               _tensor(v_t, plan.vt_shape, torch.bfloat16, "v_t"), c,
                               _tensor(o_r, ts, torch.bfloat16, "o_r"), _stream(stream)))


def sva_block_means(plan: Plan, k_t, v_t, km_t, vm_t, stream=None) -> None:
    import torch
    bf = torch.bfloat16
    _check(lib().sva_block_means(plan.handle, _tensor(k_t, plan.kt_shape, bf, "k_t"),
                                 _tensor(v_t, plan.vt_shape, bf, "v_t"),
                                 _tensor(km_t, plan.km_shape, bf, "km_t"),
                                 _tensor(vm_t, plan.vm_shape, bf, "vm_t"), _stream(stream)))


def sva_attention_compensated(plan: Plan, q_r, k_t, v_t, col, km_t, vm_t, o_r,
                              stream=None) -> None:
    import torch
    bf = torch.bfloat16
    ts = plan.tile_shape
    c = None
    if col is not None:
        c = _tensor(col, (int(plan.info.nnz),), torch.int32, "col")
    elif not plan.info.dense:
        raise ValueError("col is required for a sparse plan")
    _check(lib().sva_attention_compensated(
        plan.handle, _tensor(q_r, ts, bf, "q_r"), _tensor(k_t, plan.kt_shape, bf, "k_t"),
        _tensor(v_t, plan.vt_shape, bf, "v_t"), c, _tensor(km_t, plan.km_shape, bf, "km_t"),
        _tensor(vm_t, plan.vm_shape, bf, "vm_t"), _tensor(o_r, ts, bf, "o_r"), _stream(stream)))


def _attention_args(plan: Plan, q_r, k_t, v_t, col, km_t, vm_t, o, o_layout):
    import torch
    bf = torch.bfloat16
    c = None
    if col is not None:
        c = _tensor(col, (int(plan.info.nnz),), torch.int32, "col")
    elif not plan.info.dense:
        raise ValueError("col is required for a sparse plan")
    if (km_t is None) != (vm_t is None):
        raise ValueError("km_t and vm_t go together")
    oshape = plan.raster_shape if o_layout == SVA_LAYOUT_RASTER else plan.tile_shape
    return (plan.handle, _tensor(q_r, plan.tile_shape, bf, "q_r"),
            _tensor(k_t, plan.kt_shape, bf, "k_t"), _tensor(v_t, plan.vt_shape, bf, "v_t"), c,
            _tensor(km_t, plan.km_shape, bf, "km_t") if km_t is not None else None,
            _tensor(vm_t, plan.vm_shape, bf, "vm_t") if vm_t is not None else None,
            _tensor(o, oshape, bf, "o"), int(o_layout))


def sva_attention_ex(plan: Plan, q_r, k_t, v_t, col, km_t, vm_t, o, o_layout,
                     stream=None) -> None:
    _check(lib().sva_attention_ex(*_attention_args(plan, q_r, k_t, v_t, col, km_t, vm_t, o,
                                                   o_layout), _stream(stream)))


def sva_attention_ws(plan: Plan, q_r, k_t, v_t, col, km_t, vm_t, o, o_layout, workspace,
                     stream=None) -> None:
    """sva_attention_ex with the plan's long rows split over several
    workgroups; ``workspace`` (info.attention_workspace_bytes) holds their
    partials.  workspace None: exactly sva_attention_ex."""
    ws, ws_bytes = _workspace(workspace)
    _check(lib().sva_attention_ws(*_attention_args(plan, q_r, k_t, v_t, col, km_t, vm_t, o,
                                                   o_layout), ws, ws_bytes, _stream(stream)))


def sva_forward(plan: Plan, q, k, v, wq, wk, q_r, k_t, v_t, select_ws, col, km_t, vm_t,
                attn_ws, o, marks=None, stream=None) -> None:
    """The whole step in one call (see include/sva.h).  ``marks``: None or
    SVA_FORWARD_MARKS torch.cuda.Event objects, recorded at the stage
    boundaries; an event torch has not created yet is recorded once on the
    stream first, which creates it."""
    import torch
    bf = torch.bfloat16
    shp, wshape = plan.raster_shape, (plan.desc.H, plan.desc.d)
    sparse, comp = not plan.info.dense, plan.compensated
    if sparse and (col is None or select_ws is None):
        raise ValueError("a sparse plan needs col and select_ws")
    if comp and (km_t is None or vm_t is None):
        raise ValueError("a compensated plan needs km_t and vm_t")
    sws, sws_bytes = _workspace(select_ws if sparse else None)
    aws, aws_bytes = _workspace(attn_ws)
    b = sva_step_buffers(
        q=_tensor(q, shp, bf, "q").value, k=_tensor(k, shp, bf, "k").value,
        v=_tensor(v, shp, bf, "v").value,
        wq=_tensor(wq, wshape, torch.float32, "wq").value if wq is not None else None,
        wk=_tensor(wk, wshape, torch.float32, "wk").value if wk is not None else None,
        q_r=_tensor(q_r, plan.tile_shape, bf, "q_r").value,
        k_t=_tensor(k_t, plan.kt_shape, bf, "k_t").value,
        v_t=_tensor(v_t, plan.vt_shape, bf, "v_t").value,
        select_ws=sws.value if sws is not None else None, select_ws_bytes=sws_bytes,
        col=_tensor(col, (int(plan.info.nnz),), torch.int32, "col").value if sparse else None,
        km_t=_tensor(km_t, plan.km_shape, bf, "km_t").value if comp else None,
        vm_t=_tensor(vm_t, plan.vm_shape, bf, "vm_t").value if comp else None,
        attn_ws=aws.value if aws is not None else None, attn_ws_bytes=aws_bytes,
        o=_tensor(o, shp, bf, "o").value)
    st = _stream(stream)
    mk = None
    if marks is not None:
        if len(marks) != SVA_FORWARD_MARKS:
            raise ValueError(f"marks must hold {SVA_FORWARD_MARKS} events")
        handles = []
        for ev in marks:
            if ev.cuda_event == 0:
                ev.record(torch.cuda.current_stream() if stream is None else stream)
            handles.append(ev.cuda_event)
        mk = (ctypes.c_void_p * SVA_FORWARD_MARKS)(*handles)
    _check(lib().sva_forward(plan.handle, ctypes.byref(b), mk, st))


def sva_status_string(status: int) -> str:
    return lib().sva_status_string(status).decode()


def sva_last_error() -> str:
    return lib().sva_last_error().decode()


# --------------------------------------------------------------------------
# convenience: buffers and the whole step
# --------------------------------------------------------------------------

class Buffers:
    """Device buffers for one call of the whole step on a plan."""

    def __init__(self, plan: Plan, device="cuda"):
        import torch
        bf = torch.bfloat16
        self.qn = torch.empty(plan.raster_shape, dtype=bf, device=device)
        self.kn = torch.empty(plan.raster_shape, dtype=bf, device=device)
        self.q_r = torch.empty(plan.tile_shape, dtype=bf, device=device)
        self.k_t = torch.empty(plan.kt_shape, dtype=bf, device=device)
        self.v_t = torch.empty(plan.vt_shape, dtype=bf, device=device)
        self.o_r = torch.empty(plan.tile_shape, dtype=bf, device=device)
        self.o = torch.empty(plan.raster_shape, dtype=bf, device=device)
        nnz = int(plan.info.nnz) if not plan.info.dense else 0
        self.col = torch.empty(nnz, dtype=torch.int32, device=device) if nnz else None
        if plan.compensated:
            self.km_t = torch.empty(plan.km_shape, dtype=bf, device=device)
            self.vm_t = torch.empty(plan.vm_shape, dtype=bf, device=device)
        else:
            self.km_t = self.vm_t = None
        ws = int(plan.info.select_workspace_bytes)
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=device)
        aws = int(plan.info.attention_workspace_bytes)
        self.aws = torch.empty(aws, dtype=torch.uint8, device=device) if aws else None


def forward(plan: Plan, q, k, v, wq, wk, buf: Buffers, stream=None, marks=None):
    """The whole step in one library call (sva_forward): the prologue writes
    Q' in tile order, K' as K tiles and the block means; V is reordered into
    V tiles; blocks are ranked from the means; the attention writes O
    straight into raster order.  Returns the raster output tensor ``buf.o``."""
    sva_forward(plan, q, k, v, wq, wk, buf.q_r, buf.k_t, buf.v_t, buf.ws, buf.col, buf.km_t,
                buf.vm_t, buf.aws, buf.o, marks, stream)
    return buf.o


def forward_calls(plan: Plan, q, k, v, wq, wk, buf: Buffers, stream=None):
    """The same fused step as separate library calls."""
    sparse = not plan.info.dense
    sva_qk_norm_rope_tiled(plan, q, k, wq, wk, buf.q_r, buf.k_t,
                           buf.ws if sparse else None, stream)
    sva_reorder(plan, v, buf.v_t, SVA_FORWARD_VT, stream)
    if sparse:
        sva_select_blocks(plan, None, None, buf.ws, buf.col, stream)
    if plan.compensated:
        sva_block_means(plan, buf.k_t, buf.v_t, buf.km_t, buf.vm_t, stream)
    sva_attention_ws(plan, buf.q_r, buf.k_t, buf.v_t, buf.col, buf.km_t, buf.vm_t, buf.o,
                     SVA_LAYOUT_RASTER, buf.aws, stream)
    return buf.o


def forward_staged(plan: Plan, q, k, v, wq, wk, buf: Buffers, stream=None):
    """The same step one call per stage (raster prologue, reorders, tile-order
    attention, inverse reorder), keeping every intermediate in ``buf``."""
    sva_qk_norm_rope(plan, q, k, wq, wk, buf.qn, buf.kn, stream)
    sva_reorder(plan, buf.qn, buf.q_r, SVA_FORWARD, stream)
    sva_reorder(plan, buf.kn, buf.k_t, SVA_FORWARD_KT, stream)
    sva_reorder(plan, v, buf.v_t, SVA_FORWARD_VT, stream)
    if not plan.info.dense:
        sva_select_blocks(plan, buf.q_r, buf.k_t, buf.ws, buf.col, stream)
    if plan.compensated:
        sva_block_means(plan, buf.k_t, buf.v_t, buf.km_t, buf.vm_t, stream)
    sva_attention_ws(plan, buf.q_r, buf.k_t, buf.v_t, buf.col, buf.km_t, buf.vm_t, buf.o_r,
                     SVA_LAYOUT_TILE, buf.aws, stream)
    sva_reorder(plan, buf.o_r, buf.o, SVA_INVERSE, stream)
    return buf.o
