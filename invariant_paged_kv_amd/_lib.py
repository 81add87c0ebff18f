"""ctypes binding of libbia.so: argument marshalling and host-side shape checks.

The C functions take plain pointers; before passing tensors this module checks
that their dtype, device, contiguity and shape match what the plan and the
kernels' grids assume, so a wrong tensor is an exception here rather than an
out-of-bounds access on the GPU.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_FILE = os.path.join(_PKG, "libbia.so")

BIA_MODE_PREFILL = 0
BIA_MODE_DECODE = 1
BIA_PREFILL_SPLIT = 4096
BIA_DECODE_SPLIT = 2048
BIA_Q_TILE_ROWS = 128
BIA_KV_TILE = 64
BIA_PAGE_SIZE = 16
BIA_PLAN_STRICT_CHUNK_ALIGN = 0x1
BIA_PLAN_MLA = 0x2
BIA_MLA_QK_DIM = 576
BIA_MLA_V_DIM = 512
BIA_MLA_MAX_SPLIT = 16384

_STATUS = {0: "BIA_OK", 1: "BIA_ERR_INVALID_ARG", 2: "BIA_ERR_SHAPE",
           3: "BIA_ERR_PAGE_RANGE", 4: "BIA_ERR_WORKSPACE", 5: "BIA_ERR_UNSUPPORTED",
           6: "BIA_ERR_HIP"}

_lib = None


class BiaError(RuntimeError):
    """A non-OK status from the library, or a tensor the call cannot take."""

    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_STATUS.get(status, status)}: {message}")


def lib_path() -> str:
    return _LIB_FILE


def load_library():
    """Load libbia.so from the package directory (built by
    ``python -m invariant_paged_kv_amd.build``). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_FILE):
        raise BiaError(6, f"{_LIB_FILE} not found; build it with "
                          "`python -m invariant_paged_kv_amd.build`")
    lib = ctypes.CDLL(_LIB_FILE)
    i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    p_i32 = ctypes.POINTER(ctypes.c_int32)
    lib.bia_plan_create.restype = i32
    lib.bia_plan_create.argtypes = [i32, p_i32, p_i32, p_i32, i32, i32, i32, i32, i32,
                                    i32, i32, ctypes.c_uint32, ctypes.POINTER(vp)]
    lib.bia_plan_workspace_bytes.restype = sz
    lib.bia_plan_workspace_bytes.argtypes = [vp]
    lib.bia_plan_destroy.restype = None
    lib.bia_plan_destroy.argtypes = [vp]
    run_args = [vp, vp, vp, vp, vp, f32, vp, vp, vp, sz, vp]
    lib.bia_prefill_paged.restype = i32
    lib.bia_prefill_paged.argtypes = run_args
    lib.bia_decode_paged.restype = i32
    lib.bia_decode_paged.argtypes = run_args
    lib.bia_decode_paged_static.restype = i32
    lib.bia_decode_paged_static.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp]
    mla_args = [vp, vp, vp, vp, f32, vp, vp, vp, sz, vp]
    lib.bia_mla_prefill_paged.restype = i32
    lib.bia_mla_prefill_paged.argtypes = mla_args
    lib.bia_mla_decode_paged.restype = i32
    lib.bia_mla_decode_paged.argtypes = mla_args
    lib.bia_append_paged_kv.restype = i32
    lib.bia_append_paged_kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.bia_merge_states.restype = i32
    lib.bia_merge_states.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp]
    lib.bia_prefill_chunk_align.restype = i32
    lib.bia_prefill_chunk_align.argtypes = []
    lib.bia_last_error.restype = ctypes.c_char_p
    lib.bia_last_error.argtypes = []
    lib.bia_plan_num_items.restype = i32
    lib.bia_plan_num_items.argtypes = [vp]
    lib.bia_plan_get_items.restype = i32
    lib.bia_plan_get_items.argtypes = [vp, p_i32, i32]
    lib.bia_plan_num_states.restype = i64
    lib.bia_plan_num_states.argtypes = [vp]
    lib.bia_decode_graph_create.restype = i32
    lib.bia_decode_graph_create.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                            ctypes.POINTER(vp)]
    lib.bia_decode_graph_workspace_bytes.restype = sz
    lib.bia_decode_graph_workspace_bytes.argtypes = [vp]
    lib.bia_decode_graph_destroy.restype = None
    lib.bia_decode_graph_destroy.argtypes = [vp]
    lib.bia_decode_graph_run.restype = i32
    lib.bia_decode_graph_run.argtypes = [vp, i32, vp, vp, vp, vp, vp, f32, vp, vp, vp, sz, vp]
    lib.bia_decode_graph_read_flags.restype = i32
    lib.bia_decode_graph_read_flags.argtypes = [vp, vp, i32, p_i32, vp]
    _lib = lib
    return lib


def bia_last_error() -> str:
    return load_library().bia_last_error().decode()


def _check(status: int):
    if status != 0:
        raise BiaError(status, bia_last_error())


def _host_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _ptr_i32(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class Plan:
    """A library-owned plan (``bia_plan*``) plus the sizes needed to check the
    tensors of its runs. It may be destroyed (``close()``, or collected) as
    soon as its run calls have returned; the library reuses its pinned
    work-list block only after the device has read it."""

    def __init__(self, handle, mode, batch, num_qo_heads, num_kv_heads, head_dim,
                 num_pages, total_q, total_pages, split_size, flags=0):
        self._h = handle
        self.flags = flags
        self.mla = bool(flags & BIA_PLAN_MLA)
        self.mode = mode
        self.batch = batch
        self.num_qo_heads = num_qo_heads
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.num_pages = num_pages
        self.total_q = total_q
        self.total_pages = total_pages
        self.split_size = split_size
        self.workspace_bytes = int(load_library().bia_plan_workspace_bytes(handle))

    @property
    def handle(self):
        if self._h is None:
            raise BiaError(1, "plan already destroyed")
        return self._h

    @property
    def num_items(self) -> int:
        return int(load_library().bia_plan_num_items(self.handle))

    @property
    def num_states(self) -> int:
        return int(load_library().bia_plan_num_states(self.handle))

    def items(self) -> np.ndarray:
        """Work list, ``[num_items, 8]`` int32: q_row0, n_tok, pos0, kv_len,
        page_off, kv_head, kv_begin, state (launch order)."""
        n = self.num_items
        buf = np.zeros((n, 8), dtype=np.int32)
        if n:
            load_library().bia_plan_get_items(self.handle, _ptr_i32(buf), n)
        return buf

    def close(self):
        if self._h is not None:
            load_library().bia_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def bia_plan_create(mode, qo_indptr, kv_indptr, page_table, *, num_qo_heads,
                    num_kv_heads, head_dim, num_pages, split_size,
                    page_size: int = BIA_PAGE_SIZE, flags: int = 0) -> Plan:
    lib = load_library()
    qo = _host_i32(qo_indptr)
    kv = _host_i32(kv_indptr)
    pt = _host_i32(page_table if page_table is not None else [])
    batch = len(qo) - 1
    if len(kv) != len(qo):
        raise BiaError(2, "qo_indptr and kv_indptr differ in length")
    handle = ctypes.c_void_p()
    _check(lib.bia_plan_create(int(mode), _ptr_i32(qo), _ptr_i32(kv),
                               _ptr_i32(pt) if pt.size else None, batch,
                               num_qo_heads, num_kv_heads, head_dim, page_size,
                               num_pages, split_size, int(flags), ctypes.byref(handle)))
    kv_lens = np.diff(kv.astype(np.int64))
    total_pages = int(((kv_lens + page_size - 1) // page_size).sum()) if batch else 0
    return Plan(handle.value, int(mode), batch, num_qo_heads, num_kv_heads, head_dim,
                num_pages, int(qo[-1]) if batch else 0, total_pages, split_size, int(flags))


def bia_plan_workspace_bytes(plan: Plan) -> int:
    return int(load_library().bia_plan_workspace_bytes(plan.handle))


def bia_plan_destroy(plan: Plan):
    plan.close()


def bia_prefill_chunk_align() -> int:
    return int(load_library().bia_prefill_chunk_align())


# ------------------------------------------------------------------ tensors --

def _torch():
    import torch
    return torch


def _dev_ptr(t, name, dtype, shape=None, min_numel=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise BiaError(1, f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise BiaError(1, f"{name} must be on the GPU, got {t.device}")
    if device is not None and t.device != device:
        raise BiaError(1, f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise BiaError(1, f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise BiaError(1, f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise BiaError(2, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise BiaError(2, f"{name} has {t.numel()} elements, needs >= {min_numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _run(fn, plan: Plan, mode, q, k_pool, v_pool, page_table_dev, sm_scale, out, lse,
         workspace, stream):
    torch = _torch()
    if plan.mode != mode:
        raise BiaError(1, "plan was made for the other mode")
    if plan.mla:
        raise BiaError(1, "an MLA plan runs through bia_mla_*_paged")
    dev = q.device if isinstance(q, torch.Tensor) else None
    bf16 = torch.bfloat16
    Hq, Hkv, D = plan.num_qo_heads, plan.num_kv_heads, plan.head_dim
    qp = _dev_ptr(q, "q", bf16, (plan.total_q, Hq, D))
    pool_shape = (plan.num_pages, BIA_PAGE_SIZE, Hkv, D)
    kp = _dev_ptr(k_pool, "k_pool", bf16, pool_shape, device=dev)
    vp = _dev_ptr(v_pool, "v_pool", bf16, pool_shape, device=dev)
    ptp = _dev_ptr(page_table_dev, "page_table_dev", torch.int32,
                   min_numel=plan.total_pages, device=dev)
    op = _dev_ptr(out, "out", bf16, (plan.total_q, Hq, D), device=dev)
    lp = None if lse is None else _dev_ptr(lse, "lse", torch.float32,
                                          (plan.total_q, Hq), device=dev)
    wp = _dev_ptr(workspace, "workspace", torch.uint8, min_numel=plan.workspace_bytes,
                  device=dev)
    _check(fn(ctypes.c_void_p(plan.handle), qp, kp, vp, ptp, float(sm_scale), op, lp, wp,
              workspace.numel(), _stream_handle(stream, q.device)))


def bia_prefill_paged(plan: Plan, q, k_pool, v_pool, page_table_dev, sm_scale, out,
                      lse, workspace, stream=None):
    """Causal paged prefill (see ``bia_prefill_paged`` in bia.h)."""
    _run(load_library().bia_prefill_paged, plan, BIA_MODE_PREFILL, q, k_pool, v_pool,
         page_table_dev, sm_scale, out, lse, workspace, stream)


def bia_decode_paged(plan: Plan, q, k_pool, v_pool, page_table_dev, sm_scale, out, lse,
                     workspace, stream=None):
    """Paged decode, one query token per request (see ``bia_decode_paged``)."""
    _run(load_library().bia_decode_paged, plan, BIA_MODE_DECODE, q, k_pool, v_pool,
         page_table_dev, sm_scale, out, lse, workspace, stream)


BIA_STATIC_WORKSPACE_BYTES = 32 << 20


def bia_decode_paged_static(plan: Plan, q, k_pool, v_pool, page_table_dev, sm_scale, out,
                            lse, stream=None):
    """Paged decode with the library's static device workspace instead of a
    caller buffer (see ``bia_decode_paged_static`` in bia.h): allocates
    nothing; calls that can overlap on one GPU must not be made."""
    torch = _torch()
    if plan.mode != BIA_MODE_DECODE:
        raise BiaError(1, "plan was made for the other mode")
    if plan.mla:
        raise BiaError(1, "an MLA plan runs through bia_mla_*_paged")
    dev = q.device if isinstance(q, torch.Tensor) else None
    bf16 = torch.bfloat16
    Hq, Hkv, D = plan.num_qo_heads, plan.num_kv_heads, plan.head_dim
    qp = _dev_ptr(q, "q", bf16, (plan.total_q, Hq, D))
    pool_shape = (plan.num_pages, BIA_PAGE_SIZE, Hkv, D)
    kp = _dev_ptr(k_pool, "k_pool", bf16, pool_shape, device=dev)
    vp = _dev_ptr(v_pool, "v_pool", bf16, pool_shape, device=dev)
    ptp = _dev_ptr(page_table_dev, "page_table_dev", torch.int32,
                   min_numel=plan.total_pages, device=dev)
    op = _dev_ptr(out, "out", bf16, (plan.total_q, Hq, D), device=dev)
    lp = None if lse is None else _dev_ptr(lse, "lse", torch.float32,
                                          (plan.total_q, Hq), device=dev)
    _check(load_library().bia_decode_paged_static(ctypes.c_void_p(plan.handle), qp, kp, vp,
                                                  ptp, float(sm_scale), op, lp,
                                                  _stream_handle(stream, q.device)))


def _run_mla(fn, plan: Plan, mode, q, kv_pool, page_table_dev, sm_scale, out, lse,
             workspace, stream):
    torch = _torch()
    if plan.mode != mode:
        raise BiaError(1, "plan was made for the other mode")
    if not plan.mla:
        raise BiaError(1, "plan was not made with BIA_PLAN_MLA")
    dev = q.device if isinstance(q, torch.Tensor) else None
    bf16 = torch.bfloat16
    Hq = plan.num_qo_heads
    qp = _dev_ptr(q, "q", bf16, (plan.total_q, Hq, BIA_MLA_QK_DIM))
    kvp = _dev_ptr(kv_pool, "kv_pool", bf16, (plan.num_pages, BIA_PAGE_SIZE, BIA_MLA_QK_DIM),
                   device=dev)
    ptp = _dev_ptr(page_table_dev, "page_table_dev", torch.int32,
                   min_numel=plan.total_pages, device=dev)
    op = _dev_ptr(out, "out", bf16, (plan.total_q, Hq, BIA_MLA_V_DIM), device=dev)
    lp = None if lse is None else _dev_ptr(lse, "lse", torch.float32,
                                          (plan.total_q, Hq), device=dev)
    wp = _dev_ptr(workspace, "workspace", torch.uint8, min_numel=plan.workspace_bytes,
                  device=dev)
    _check(fn(ctypes.c_void_p(plan.handle), qp, kvp, ptp, float(sm_scale), op, lp, wp,
              workspace.numel(), _stream_handle(stream, q.device)))


def bia_mla_prefill_paged(plan: Plan, q, kv_pool, page_table_dev, sm_scale, out, lse,
                          workspace, stream=None):
    """Causal latent (MLA) prefill over a paged latent cache (see
    ``bia_mla_prefill_paged`` in bia.h)."""
    _run_mla(load_library().bia_mla_prefill_paged, plan, BIA_MODE_PREFILL, q, kv_pool,
             page_table_dev, sm_scale, out, lse, workspace, stream)


def bia_mla_decode_paged(plan: Plan, q, kv_pool, page_table_dev, sm_scale, out, lse,
                         workspace, stream=None):
    """Latent (MLA) decode, one query token per request (see
    ``bia_mla_decode_paged``)."""
    _run_mla(load_library().bia_mla_decode_paged, plan, BIA_MODE_DECODE, q, kv_pool,
             page_table_dev, sm_scale, out, lse, workspace, stream)


def bia_append_paged_kv(plan: Plan, k_new, v_new, page_table_dev, k_pool, v_pool,
                        workspace, stream=None):
    """Write each request's new tokens' K and V into their page slots (see
    ``bia_append_paged_kv`` in bia.h). ``k_new``/``v_new`` are bf16
    ``[sum qo_len, Hkv, D]``; the pools are written in place."""
    torch = _torch()
    dev = k_new.device if isinstance(k_new, torch.Tensor) else None
    bf16 = torch.bfloat16
    Hkv, D = plan.num_kv_heads, plan.head_dim
    kn = _dev_ptr(k_new, "k_new", bf16, (plan.total_q, Hkv, D))
    vn = _dev_ptr(v_new, "v_new", bf16, (plan.total_q, Hkv, D), device=dev)
    pool_shape = (plan.num_pages, BIA_PAGE_SIZE, Hkv, D)
    kp = _dev_ptr(k_pool, "k_pool", bf16, pool_shape, device=dev)
    vp = _dev_ptr(v_pool, "v_pool", bf16, pool_shape, device=dev)
    ptp = _dev_ptr(page_table_dev, "page_table_dev", torch.int32,
                   min_numel=plan.total_pages, device=dev)
    wp = _dev_ptr(workspace, "workspace", torch.uint8, min_numel=plan.workspace_bytes,
                  device=dev)
    _check(load_library().bia_append_paged_kv(ctypes.c_void_p(plan.handle), kn, vn, ptp, kp,
                                              vp, wp, workspace.numel(),
                                              _stream_handle(stream, k_new.device)))


def bia_merge_states(v, s, state_indptr_dev, out, out_lse=None, stream=None):
    """Fixed-order merge of partial states (see ``bia_merge_states``).

    ``v [n_states, H, D]`` fp32, ``s [n_states, H]`` fp32 (natural-log lse,
    -inf = empty), ``state_indptr_dev [n_rows + 1]`` int32 on the GPU,
    ``out [n_rows, H, D]`` bf16, ``out_lse [n_rows, H]`` fp32 or None.
    """
    torch = _torch()
    lib = load_library()
    if v.dim() != 3:
        raise BiaError(2, "v must be [n_states, H, D]")
    n_states, H, D = v.shape
    n_rows = state_indptr_dev.numel() - 1
    dev = v.device
    vp_ = _dev_ptr(v, "v", torch.float32)
    sp = _dev_ptr(s, "s", torch.float32, (n_states, H), device=dev)
    ip = _dev_ptr(state_indptr_dev, "state_indptr_dev", torch.int32, device=dev)
    op = _dev_ptr(out, "out", torch.bfloat16, (n_rows, H, D), device=dev)
    lp = None if out_lse is None else _dev_ptr(out_lse, "out_lse", torch.float32,
                                              (n_rows, H), device=dev)
    _check(lib.bia_merge_states(vp_, sp, ip, n_rows, H, D, op, lp,
                                _stream_handle(stream, dev)))


# ------------------------------------------------------- graph-capturable --

class DecodeGraph:
    """A fixed-capacity decode planned on the device (``bia_decode_graph*``):
    its runs make no host-to-device copy and allocate nothing, so they can be
    captured in a HIP graph and replayed with new buffer contents."""

    def __init__(self, handle, max_batch, num_qo_heads, num_kv_heads, head_dim, num_pages,
                 max_kv_len, page_table_capacity, split_size):
        self._h = handle
        self.max_batch = max_batch
        self.num_qo_heads = num_qo_heads
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.num_pages = num_pages
        self.max_kv_len = max_kv_len
        self.page_table_capacity = page_table_capacity
        self.split_size = split_size
        self.workspace_bytes = int(load_library().bia_decode_graph_workspace_bytes(handle))

    @property
    def handle(self):
        if self._h is None:
            raise BiaError(1, "decode graph already destroyed")
        return self._h

    def close(self):
        if self._h is not None:
            load_library().bia_decode_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def bia_decode_graph_create(*, max_batch, num_qo_heads, num_kv_heads, head_dim, num_pages,
                            max_kv_len, page_table_capacity, split_size=BIA_DECODE_SPLIT,
                            page_size: int = BIA_PAGE_SIZE) -> DecodeGraph:
    handle = ctypes.c_void_p()
    _check(load_library().bia_decode_graph_create(
        max_batch, num_qo_heads, num_kv_heads, head_dim, page_size, num_pages, max_kv_len,
        page_table_capacity, split_size, ctypes.byref(handle)))
    return DecodeGraph(handle.value, max_batch, num_qo_heads, num_kv_heads, head_dim,
                       num_pages, max_kv_len, page_table_capacity, split_size)


def bia_decode_graph_workspace_bytes(dg: DecodeGraph) -> int:
    return int(load_library().bia_decode_graph_workspace_bytes(dg.handle))


def bia_decode_graph_destroy(dg: DecodeGraph):
    dg.close()


def bia_decode_graph_run(dg: DecodeGraph, batch, kv_indptr_dev, q, k_pool, v_pool,
                         page_table_dev, sm_scale, out, lse, workspace, stream=None):
    """Decode of ``batch`` requests without host planning (see
    ``bia_decode_graph_run`` in bia.h). ``kv_indptr_dev`` is a device int32
    tensor of ``batch + 1`` cumulative kv lengths; ``page_table_dev`` holds at
    least ``page_table_capacity`` entries."""
    torch = _torch()
    if not 0 <= batch <= dg.max_batch:
        raise BiaError(2, f"batch {batch} outside [0, {dg.max_batch}]")
    dev = q.device if isinstance(q, torch.Tensor) else None
    bf16 = torch.bfloat16
    Hq, Hkv, D = dg.num_qo_heads, dg.num_kv_heads, dg.head_dim
    ip = _dev_ptr(kv_indptr_dev, "kv_indptr_dev", torch.int32, (batch + 1,), device=dev)
    qp = _dev_ptr(q, "q", bf16, (batch, Hq, D), device=dev)
    pool_shape = (dg.num_pages, BIA_PAGE_SIZE, Hkv, D)
    kp = _dev_ptr(k_pool, "k_pool", bf16, pool_shape, device=dev)
    vp = _dev_ptr(v_pool, "v_pool", bf16, pool_shape, device=dev)
    ptp = _dev_ptr(page_table_dev, "page_table_dev", torch.int32,
                   min_numel=dg.page_table_capacity, device=dev)
    op = _dev_ptr(out, "out", bf16, (batch, Hq, D), device=dev)
    lp = None if lse is None else _dev_ptr(lse, "lse", torch.float32, (batch, Hq), device=dev)
    wp = _dev_ptr(workspace, "workspace", torch.uint8, min_numel=dg.workspace_bytes,
                  device=dev)
    _check(load_library().bia_decode_graph_run(
        ctypes.c_void_p(dg.handle), batch, ip, qp, kp, vp, ptp, float(sm_scale), op, lp, wp,
        workspace.numel(), _stream_handle(stream, q.device)))


def bia_decode_graph_read_flags(dg: DecodeGraph, workspace, batch, stream=None) -> np.ndarray:
    """Per-request flags of the last run on ``workspace`` (0 = valid; 1 kv_len
    out of range, 2 pages past the table capacity, 4 a page id outside the
    pool). Waits for the stream."""
    torch = _torch()
    flags = np.zeros(max(batch, 1), dtype=np.int32)
    wp = _dev_ptr(workspace, "workspace", torch.uint8, min_numel=dg.workspace_bytes)
    _check(load_library().bia_decode_graph_read_flags(
        ctypes.c_void_p(dg.handle), wp, batch, _ptr_i32(flags),
        _stream_handle(stream, workspace.device)))
    return flags[:batch]
