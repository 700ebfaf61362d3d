"""Python binding of libep_hip (include/ep.h): argument marshalling only.

Every computation runs in the library's HIP kernels.  torch supplies device
memory (tensors) and the stream (``torch.cuda.current_stream()``); the
functions below check dtypes / shapes / devices, pass raw pointers through
ctypes and turn a negative status into ``RuntimeError``.  If the built
library is missing, loading raises immediately: there is no fallback path.

The C entry points keep their names (``ep_dispatch_layout``, ``ep_dispatch``,
``ep_combine``, ...); ``dispatch_layout`` / ``dispatch`` / ``combine`` are the
same calls with outputs allocated as torch tensors.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# EP_HIP_LIB: another build of the library to load (the CPU suite's
# sanitizer run uses one built with host-side address / UB sanitizers)
LIB_PATH = os.environ.get("EP_HIP_LIB") or os.path.join(_PKG, "libep_hip.so")

EP_FMT_BF16, EP_FMT_FP8_S128, EP_FMT_MXFP8, EP_FMT_NVFP4 = 0, 1, 2, 3
EP_OK, EP_EINVAL, EP_EALIGN, EP_EWORKSPACE, EP_EHIP, EP_EDEVICE = 0, -1, -2, -3, -4, -5
EP_STATIC_SCRATCH_BYTES = 16 << 20   # the static scratch of ep_dispatch_with_layout_static
# device error flags (ep_check): bad expert id, internal slot check, RANK_MAJOR overflow, stale plan
EP_ERRFLAG_BAD_EXPERT, EP_ERRFLAG_BAD_SLOT, EP_ERRFLAG_RANK_OVERFLOW, EP_ERRFLAG_STALE_PLAN = 0x1, 0x2, 0x4, 0x8

# every symbol include/ep.h declares
EXPORTED = (
    "ep_abi_version", "ep_strerror", "ep_validate_shape", "ep_workspace_bytes", "ep_workspace_init",
    "ep_dispatch_layout", "ep_dispatch", "ep_dispatch_from_layout", "ep_dispatch_with_layout", "ep_dispatch_cached",
    "ep_dispatch_ranks_cached", "ep_dispatch_ranks_with_layout", "ep_combine", "ep_check",
    "ep_dispatch_ranks", "ep_expert_reduce_ranks", "ep_combine_ranks", "ep_quant_fp8_s128",
    "ep_expert_scale_bf16", "ep_expert_requant_mxfp8", "ep_expert_requant_nvfp4", "ep_accounting",
    "ep_calib_copy", "ep_stream", "ep_dispatch_with_layout_static", "ep_plan_info",
)


class ep_shape(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("hidden", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_ranks", ctypes.c_int32),
        ("num_nodes", ctypes.c_int32),
        ("num_topk", ctypes.c_int32),
        ("x_format", ctypes.c_int32),
        ("y_format", ctypes.c_int32),
        ("rank_capacity", ctypes.c_int32),
        ("rank_rows", ctypes.c_int32),
    ]

    @property
    def rows(self) -> int:
        """Receive rows: T*k (compacted) or R * rank_capacity (RANK_MAJOR)."""
        if self.rank_capacity > 0:
            return self.num_ranks * self.rank_capacity
        return self.num_tokens * self.num_topk

    @property
    def rank_rows_cap(self) -> int:
        """Receive rows of the (token, rank) layout: T * min(k, R)."""
        return self.num_tokens * min(self.num_topk, self.num_ranks)


class ep_accounting_t(ctypes.Structure):
    _fields_ = [
        ("rdma_algo_tokens", ctypes.c_int64),
        ("rdma_physical_tokens", ctypes.c_double),
        ("rdma_physical_tokens_exact", ctypes.c_int64),
        ("nvl_tokens", ctypes.c_int64),
        ("dispatch_rdma_bytes_bf16", ctypes.c_double),
        ("dispatch_nvl_bytes_bf16", ctypes.c_double),
        ("combine_rdma_bytes_bf16", ctypes.c_double),
        ("combine_nvl_bytes_bf16", ctypes.c_double),
        ("fp8_factor", ctypes.c_double),
        ("dispatch_rdma_bytes_fp8", ctypes.c_double),
        ("dispatch_nvl_bytes_fp8", ctypes.c_double),
        ("hbm_layout_bytes", ctypes.c_double),
        ("hbm_dispatch_bytes", ctypes.c_double),
        ("hbm_combine_bytes", ctypes.c_double),
        ("hbm_dispatch_ranks_bytes", ctypes.c_double),
        ("hbm_combine_ranks_bytes", ctypes.c_double),
    ] + [(f"hbm_{call}_{rw}_bytes", ctypes.c_double)
         for call in ("layout", "dispatch", "combine", "dispatch_ranks", "combine_ranks") for rw in ("read", "write")]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class ep_plan_info_t(ctypes.Structure):
    _fields_ = [
        ("workspace_bytes", ctypes.c_size_t),
        ("region_offset", ctypes.c_size_t * 8),
        ("region_bytes", ctypes.c_size_t * 8),
        ("tiles", ctypes.c_int32),
        ("tile_tokens", ctypes.c_int32),
        ("tile_waves", ctypes.c_int32),
        ("count_threads", ctypes.c_int32),
        ("count_lds_bytes", ctypes.c_size_t),
        ("single_launch_lds_bytes", ctypes.c_size_t),
        ("single_launch_threads", ctypes.c_int32),
        ("scan_copy_lds_bytes", ctypes.c_size_t),
    ]

    def as_dict(self):
        out = {}
        for name, _ in self._fields_:
            v = getattr(self, name)
            out[name] = list(v) if isinstance(v, ctypes.Array) else v
        return out


_lib = None


def load():
    """Load libep_hip.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (__graft_entry__.build() or "
                           "python combine_dispatch_layout_02_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    SP = ctypes.POINTER(ep_shape)
    sig = {
        "ep_abi_version": (ctypes.c_int, []),
        "ep_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "ep_validate_shape": (ctypes.c_int, [SP]),
        "ep_workspace_bytes": (ctypes.c_int, [SP, ctypes.POINTER(sz)]),
        "ep_workspace_init": (ctypes.c_int, [P, sz, P]),
        "ep_dispatch_layout": (ctypes.c_int, [SP, P, P, P, P, P, P, P, sz, P]),
        "ep_dispatch": (ctypes.c_int, [SP, P, P, P, P, P, P, P, P, P, P, P, sz, P]),
        "ep_dispatch_from_layout": (ctypes.c_int, [SP, P, P, P, P, P, P, P, P, P, P, P, sz, P]),
        "ep_dispatch_with_layout": (ctypes.c_int, [SP] + [P] * 15 + [P, sz, P]),
        "ep_dispatch_cached": (ctypes.c_int, [SP, P, P, P, P, P, P]),
        "ep_dispatch_ranks_cached": (ctypes.c_int, [SP, P, P, P, P, P, P]),
        "ep_dispatch_ranks_with_layout": (ctypes.c_int, [SP] + [P] * 16 + [P, sz, P]),
        "ep_combine": (ctypes.c_int, [SP, P, P, P, P, P, P]),
        "ep_dispatch_ranks": (ctypes.c_int, [SP, P, P, P, P, P, P, P, P, P, P, P, P, sz, P]),
        "ep_expert_reduce_ranks": (ctypes.c_int, [SP, P, P, P, P, P, P, P, P]),
        "ep_combine_ranks": (ctypes.c_int, [SP, P, P, P, P]),
        "ep_check": (ctypes.c_int, [P, sz, P, ctypes.POINTER(ctypes.c_uint32)]),
        "ep_quant_fp8_s128": (ctypes.c_int, [i64, i32, P, P, P, P]),
        "ep_expert_scale_bf16": (ctypes.c_int, [SP, P, P, P, P, P]),
        "ep_expert_requant_mxfp8": (ctypes.c_int, [SP, P, P, P, P, P, P, P]),
        "ep_expert_requant_nvfp4": (ctypes.c_int, [SP, P, P, P, P, P, P]),
        "ep_accounting": (ctypes.c_int, [SP, i32, P, P, i64, i64, ctypes.POINTER(ep_accounting_t)]),
        "ep_calib_copy": (ctypes.c_int, [P, P, sz, P]),
        "ep_stream": (ctypes.c_int, [i32, P, P, sz, sz, i32, P]),
        "ep_dispatch_with_layout_static": (ctypes.c_int, [SP] + [P] * 15 + [P]),
        "ep_plan_info": (ctypes.c_int, [SP, ctypes.POINTER(ep_plan_info_t)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.ep_abi_version() != 8:
        raise RuntimeError("libep_hip ABI version mismatch")
    _lib = lib
    return lib


def plan_info(shape: ep_shape) -> dict:
    """ep_plan_info: workspace regions, plan tiling and LDS per launch (host only)."""
    info = ep_plan_info_t()
    _ok(load().ep_plan_info(ctypes.byref(shape), ctypes.byref(info)), "ep_plan_info")
    return info.as_dict()


def strerror(rc: int) -> str:
    return load().ep_strerror(rc).decode()


def _ok(rc: int, what: str):
    if rc != EP_OK:
        raise RuntimeError(f"{what} failed: {strerror(rc)} ({rc})")


def make_shape(T, H, E, R, N, k, x_format=EP_FMT_BF16, y_format=EP_FMT_BF16, rank_capacity=0,
               rank_rows=0) -> ep_shape:
    return ep_shape(int(T), int(H), int(E), int(R), int(N), int(k), int(x_format), int(y_format),
                    int(rank_capacity), int(rank_rows))


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return ctypes.c_void_p(int(t))
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


# --------------------------------------------------------------------------- workspace

class Workspace:
    """Device workspace for one shape (allocated once, zeroed by the library)."""

    def __init__(self, shape: ep_shape, device=None, stream=None):
        lib = load()
        n = ctypes.c_size_t()
        _ok(lib.ep_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)), "ep_workspace_bytes")
        self.nbytes = int(n.value)
        dev = torch.device("cuda") if device is None else torch.device(device)
        self._buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=dev)
        off = (-self._buf.data_ptr()) % 256
        self.tensor = self._buf[off:off + self.nbytes]
        self.planned_for = None   # (topk_idx pointer, shape fields) of the last layout call
        _ok(lib.ep_workspace_init(_ptr(self.tensor), self.nbytes, _stream(stream)), "ep_workspace_init")

    @property
    def ptr(self):
        return _ptr(self.tensor)

    def check(self, stream=None) -> int:
        """Synchronize and read/clear the device error word (raises on a flag)."""
        flags = ctypes.c_uint32()
        rc = load().ep_check(self.ptr, self.nbytes, _stream(stream), ctypes.byref(flags))
        if rc == EP_EDEVICE:
            raise RuntimeError(f"ep_check: {strerror(rc)} (flags {flags.value:#x})")
        _ok(rc, "ep_check")
        return flags.value


# --------------------------------------------------------------------------- C-named calls

def ep_dispatch_layout(shape, topk_idx, num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank,
                       num_tokens_per_node, rdma_algo_token_count, ws: Workspace, stream=None):
    T, k, R, E, N = shape.num_tokens, shape.num_topk, shape.num_ranks, shape.num_experts, shape.num_nodes
    _need(topk_idx, torch.int64, (T, k), "topk_idx")
    _need(num_tokens_per_rank, torch.int32, (R,), "num_tokens_per_rank")
    _need(num_tokens_per_expert, torch.int32, (E,), "num_tokens_per_expert")
    _need(is_token_in_rank, torch.uint8, (T, R), "is_token_in_rank")
    _need(num_tokens_per_node, torch.int32, (N,), "num_tokens_per_node")
    _need(rdma_algo_token_count, torch.int64, (1,), "rdma_algo_token_count")
    _ok(load().ep_dispatch_layout(ctypes.byref(shape), _ptr(topk_idx), _ptr(num_tokens_per_rank),
                                  _ptr(num_tokens_per_expert), _ptr(is_token_in_rank),
                                  _ptr(num_tokens_per_node), _ptr(rdma_algo_token_count), ws.ptr,
                                  ws.nbytes, _stream(stream)), "ep_dispatch_layout")
    ws.planned_for = (topk_idx.data_ptr(), _shape_key(shape))


def _shape_key(shape):
    return tuple(getattr(shape, f) for f, _ in shape._fields_)


def ep_dispatch(shape, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales, recv_src_idx, recv_topk_w,
                token_slot, expert_offset, ws: Workspace, stream=None, from_layout=False):
    """from_layout=True calls ep_dispatch_from_layout: the plan of the preceding
    ep_dispatch_layout call on this workspace and this topk_idx is reused."""
    T, k, H, E = shape.num_tokens, shape.num_topk, shape.hidden, shape.num_experts
    fp8 = shape.x_format == EP_FMT_FP8_S128
    _need(x, torch.uint8 if fp8 else torch.bfloat16, (T, H), "x")
    _need(topk_idx, torch.int64, (T, k), "topk_idx")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    rows = shape.rows
    _need(recv_x, x.dtype, (rows, H), "recv_x")
    if fp8:
        _need(x_scales, torch.float32, (T, H // 128), "x_scales")
        _need(recv_x_scales, torch.float32, (rows, H // 128), "recv_x_scales")
    _need(recv_src_idx, torch.int32, (rows,), "recv_src_idx")
    _need(recv_topk_w, torch.float32, (rows,), "recv_topk_w")
    _need(token_slot, torch.int32, (T, k), "token_slot")
    _need(expert_offset, torch.int32, (E + 1,), "expert_offset")
    fn = load().ep_dispatch
    if from_layout:
        if ws.planned_for != (topk_idx.data_ptr(), _shape_key(shape)):
            raise RuntimeError("ep_dispatch_from_layout needs a preceding ep_dispatch_layout on this "
                               "workspace with the same topk_idx and shape")
        fn = load().ep_dispatch_from_layout
    else:
        ws.planned_for = None   # ep_dispatch rewrites the plan (same content for the same topk_idx)
    _ok(fn(ctypes.byref(shape), _ptr(x), _ptr(x_scales), _ptr(topk_idx), _ptr(topk_w),
           _ptr(recv_x), _ptr(recv_x_scales), _ptr(recv_src_idx), _ptr(recv_topk_w),
           _ptr(token_slot), _ptr(expert_offset), ws.ptr, ws.nbytes, _stream(stream)),
        "ep_dispatch_from_layout" if from_layout else "ep_dispatch")


def _check_with_layout(shape, x, x_scales, topk_idx, topk_w, num_tokens_per_rank, num_tokens_per_expert,
                       is_token_in_rank, num_tokens_per_node, rdma_algo_token_count, recv_x, recv_x_scales,
                       recv_src_idx, recv_topk_w, token_slot, expert_offset):
    T, k, H, E, R, N = (shape.num_tokens, shape.num_topk, shape.hidden, shape.num_experts, shape.num_ranks,
                        shape.num_nodes)
    fp8 = shape.x_format == EP_FMT_FP8_S128
    rows = shape.rows
    _need(x, torch.uint8 if fp8 else torch.bfloat16, (T, H), "x")
    _need(topk_idx, torch.int64, (T, k), "topk_idx")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(num_tokens_per_rank, torch.int32, (R,), "num_tokens_per_rank")
    _need(num_tokens_per_expert, torch.int32, (E,), "num_tokens_per_expert")
    _need(is_token_in_rank, torch.uint8, (T, R), "is_token_in_rank")
    _need(num_tokens_per_node, torch.int32, (N,), "num_tokens_per_node")
    _need(rdma_algo_token_count, torch.int64, (1,), "rdma_algo_token_count")
    _need(recv_x, x.dtype, (rows, H), "recv_x")
    if fp8:
        _need(x_scales, torch.float32, (T, H // 128), "x_scales")
        _need(recv_x_scales, torch.float32, (rows, H // 128), "recv_x_scales")
    _need(recv_src_idx, torch.int32, (rows,), "recv_src_idx")
    _need(recv_topk_w, torch.float32, (rows,), "recv_topk_w")
    _need(token_slot, torch.int32, (T, k), "token_slot")
    _need(expert_offset, torch.int32, (E + 1,), "expert_offset")


def ep_dispatch_with_layout(shape, x, x_scales, topk_idx, topk_w, num_tokens_per_rank, num_tokens_per_expert,
                            is_token_in_rank, num_tokens_per_node, rdma_algo_token_count, recv_x, recv_x_scales,
                            recv_src_idx, recv_topk_w, token_slot, expert_offset, ws: Workspace, stream=None):
    """Layout and dispatch in one call (one launch for batches of <= 2048 pairs)."""
    _check_with_layout(shape, x, x_scales, topk_idx, topk_w, num_tokens_per_rank, num_tokens_per_expert,
                       is_token_in_rank, num_tokens_per_node, rdma_algo_token_count, recv_x, recv_x_scales,
                       recv_src_idx, recv_topk_w, token_slot, expert_offset)
    ws.planned_for = None   # no reusable plan is left in the workspace
    _ok(load().ep_dispatch_with_layout(ctypes.byref(shape), _ptr(x), _ptr(x_scales), _ptr(topk_idx), _ptr(topk_w),
                                       _ptr(num_tokens_per_rank), _ptr(num_tokens_per_expert),
                                       _ptr(is_token_in_rank), _ptr(num_tokens_per_node),
                                       _ptr(rdma_algo_token_count), _ptr(recv_x), _ptr(recv_x_scales),
                                       _ptr(recv_src_idx), _ptr(recv_topk_w), _ptr(token_slot),
                                       _ptr(expert_offset), ws.ptr, ws.nbytes, _stream(stream)),
        "ep_dispatch_with_layout")


def ep_dispatch_with_layout_static(shape, x, x_scales, topk_idx, topk_w, num_tokens_per_rank,
                                   num_tokens_per_expert, is_token_in_rank, num_tokens_per_node,
                                   rdma_algo_token_count, recv_x, recv_x_scales, recv_src_idx, recv_topk_w,
                                   token_slot, expert_offset, stream=None):
    """ep_dispatch_with_layout without a workspace: the library's static
    per-GPU scratch holds the plan (no device allocation anywhere)."""
    _check_with_layout(shape, x, x_scales, topk_idx, topk_w, num_tokens_per_rank, num_tokens_per_expert,
                       is_token_in_rank, num_tokens_per_node, rdma_algo_token_count, recv_x, recv_x_scales,
                       recv_src_idx, recv_topk_w, token_slot, expert_offset)
    _ok(load().ep_dispatch_with_layout_static(
        ctypes.byref(shape), _ptr(x), _ptr(x_scales), _ptr(topk_idx), _ptr(topk_w), _ptr(num_tokens_per_rank),
        _ptr(num_tokens_per_expert), _ptr(is_token_in_rank), _ptr(num_tokens_per_node),
        _ptr(rdma_algo_token_count), _ptr(recv_x), _ptr(recv_x_scales), _ptr(recv_src_idx), _ptr(recv_topk_w),
        _ptr(token_slot), _ptr(expert_offset), _stream(stream)), "ep_dispatch_with_layout_static")


def check_static(stream=None) -> int:
    """Synchronize and read/clear the error word of the current device's
    static scratch (ep_check with no workspace; raises on a flag)."""
    flags = ctypes.c_uint32()
    rc = load().ep_check(None, 0, _stream(stream), ctypes.byref(flags))
    if rc == EP_EDEVICE:
        raise RuntimeError(f"ep_check: {strerror(rc)} (flags {flags.value:#x})")
    _ok(rc, "ep_check")
    return flags.value


def ep_dispatch_cached(shape, x, x_scales, token_slot, recv_x, recv_x_scales=None, stream=None):
    """Rows of a previous dispatch's handle (token_slot [T, k]) for another tensor x."""
    T, k, H = shape.num_tokens, shape.num_topk, shape.hidden
    fp8 = shape.x_format == EP_FMT_FP8_S128
    _need(x, torch.uint8 if fp8 else torch.bfloat16, (T, H), "x")
    _need(token_slot, torch.int32, (T, k), "token_slot")
    _need(recv_x, x.dtype, (shape.rows, H), "recv_x")
    if fp8:
        _need(x_scales, torch.float32, (T, H // 128), "x_scales")
        _need(recv_x_scales, torch.float32, (shape.rows, H // 128), "recv_x_scales")
    _ok(load().ep_dispatch_cached(ctypes.byref(shape), _ptr(x), _ptr(x_scales), _ptr(token_slot), _ptr(recv_x),
                                  _ptr(recv_x_scales), _stream(stream)), "ep_dispatch_cached")


def ep_dispatch_ranks_cached(shape, x, x_scales, token_rank_slot, recv_x, recv_x_scales=None, stream=None):
    """Rows of a previous (token, rank) dispatch's handle (token_rank_slot [T, R]) for another tensor x."""
    T, H, R = shape.num_tokens, shape.hidden, shape.num_ranks
    fp8 = shape.x_format == EP_FMT_FP8_S128
    cap = shape.rank_rows_cap
    _need(x, torch.uint8 if fp8 else torch.bfloat16, (T, H), "x")
    _need(token_rank_slot, torch.int32, (T, R), "token_rank_slot")
    _need(recv_x, x.dtype, (cap, H), "recv_x")
    if fp8:
        _need(x_scales, torch.float32, (T, H // 128), "x_scales")
        _need(recv_x_scales, torch.float32, (cap, H // 128), "recv_x_scales")
    _ok(load().ep_dispatch_ranks_cached(ctypes.byref(shape), _ptr(x), _ptr(x_scales), _ptr(token_rank_slot),
                                        _ptr(recv_x), _ptr(recv_x_scales), _stream(stream)),
        "ep_dispatch_ranks_cached")


def ep_combine(shape, expert_out, expert_out_scales, token_slot, topk_w, y, stream=None):
    T, k, H = shape.num_tokens, shape.num_topk, shape.hidden
    fmt = shape.y_format
    if fmt == EP_FMT_MXFP8:
        _need(expert_out, torch.uint8, (shape.rows, H), "expert_out")
        _need(expert_out_scales, torch.uint8, (shape.rows, H // 32), "expert_out_scales")
    elif fmt == EP_FMT_NVFP4:
        _need(expert_out, torch.uint8, (shape.rows, H // 2), "expert_out")
        if expert_out_scales is None or expert_out_scales.dtype not in (torch.int16, torch.bfloat16) \
                or tuple(expert_out_scales.shape) != (shape.rows, H // 16):
            raise ValueError("expert_out_scales: expected bf16 bits [rows, H/16]")
    else:
        _need(expert_out, torch.bfloat16, (shape.rows, H), "expert_out")
    _need(token_slot, torch.int32, (T, k), "token_slot")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(y, torch.bfloat16, (T, H), "y")
    _ok(load().ep_combine(ctypes.byref(shape), _ptr(expert_out), _ptr(expert_out_scales), _ptr(token_slot),
                          _ptr(topk_w), _ptr(y), _stream(stream)), "ep_combine")


def ep_dispatch_ranks(shape, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales, recv_src_idx,
                      recv_topk_idx, recv_topk_w, token_rank_slot, rank_offset, ws: Workspace, stream=None):
    """(token, rank) rows from the plan of the preceding ep_dispatch_layout on
    this workspace with this topk_idx (shape.rank_rows must be 1)."""
    T, k, H, R = shape.num_tokens, shape.num_topk, shape.hidden, shape.num_ranks
    fp8 = shape.x_format == EP_FMT_FP8_S128
    cap = shape.rank_rows_cap
    _need(x, torch.uint8 if fp8 else torch.bfloat16, (T, H), "x")
    _need(topk_idx, torch.int64, (T, k), "topk_idx")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(recv_x, x.dtype, (cap, H), "recv_x")
    if fp8:
        _need(x_scales, torch.float32, (T, H // 128), "x_scales")
        _need(recv_x_scales, torch.float32, (cap, H // 128), "recv_x_scales")
    _need(recv_src_idx, torch.int32, (cap,), "recv_src_idx")
    _need(recv_topk_idx, torch.int32, (cap, k), "recv_topk_idx")
    _need(recv_topk_w, torch.float32, (cap, k), "recv_topk_w")
    _need(token_rank_slot, torch.int32, (T, R), "token_rank_slot")
    _need(rank_offset, torch.int32, (R + 1,), "rank_offset")
    if ws.planned_for != (topk_idx.data_ptr(), _shape_key(shape)):
        raise RuntimeError("ep_dispatch_ranks needs a preceding ep_dispatch_layout on this workspace "
                           "with the same topk_idx and shape")
    _ok(load().ep_dispatch_ranks(ctypes.byref(shape), _ptr(x), _ptr(x_scales), _ptr(topk_idx), _ptr(topk_w),
                                 _ptr(recv_x), _ptr(recv_x_scales), _ptr(recv_src_idx), _ptr(recv_topk_idx),
                                 _ptr(recv_topk_w), _ptr(token_rank_slot), _ptr(rank_offset), ws.ptr,
                                 ws.nbytes, _stream(stream)), "ep_dispatch_ranks")


def ep_dispatch_ranks_with_layout(shape, x, x_scales, topk_idx, topk_w, num_tokens_per_rank,
                                  num_tokens_per_expert, is_token_in_rank, num_tokens_per_node,
                                  rdma_algo_token_count, recv_x, recv_x_scales, recv_src_idx, recv_topk_idx,
                                  recv_topk_w, token_rank_slot, rank_offset, ws: Workspace, stream=None):
    """Layout and (token, rank) dispatch in one call (one launch for batches of <= 2048 pairs)."""
    T, k, H, E, R, N = (shape.num_tokens, shape.num_topk, shape.hidden, shape.num_experts, shape.num_ranks,
                        shape.num_nodes)
    fp8 = shape.x_format == EP_FMT_FP8_S128
    cap = shape.rank_rows_cap
    _need(x, torch.uint8 if fp8 else torch.bfloat16, (T, H), "x")
    _need(topk_idx, torch.int64, (T, k), "topk_idx")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(num_tokens_per_rank, torch.int32, (R,), "num_tokens_per_rank")
    _need(num_tokens_per_expert, torch.int32, (E,), "num_tokens_per_expert")
    _need(is_token_in_rank, torch.uint8, (T, R), "is_token_in_rank")
    _need(num_tokens_per_node, torch.int32, (N,), "num_tokens_per_node")
    _need(rdma_algo_token_count, torch.int64, (1,), "rdma_algo_token_count")
    _need(recv_x, x.dtype, (cap, H), "recv_x")
    if fp8:
        _need(x_scales, torch.float32, (T, H // 128), "x_scales")
        _need(recv_x_scales, torch.float32, (cap, H // 128), "recv_x_scales")
    _need(recv_src_idx, torch.int32, (cap,), "recv_src_idx")
    _need(recv_topk_idx, torch.int32, (cap, k), "recv_topk_idx")
    _need(recv_topk_w, torch.float32, (cap, k), "recv_topk_w")
    _need(token_rank_slot, torch.int32, (T, R), "token_rank_slot")
    _need(rank_offset, torch.int32, (R + 1,), "rank_offset")
    ws.planned_for = None   # no reusable plan is left in the workspace
    _ok(load().ep_dispatch_ranks_with_layout(
        ctypes.byref(shape), _ptr(x), _ptr(x_scales), _ptr(topk_idx), _ptr(topk_w), _ptr(num_tokens_per_rank),
        _ptr(num_tokens_per_expert), _ptr(is_token_in_rank), _ptr(num_tokens_per_node), _ptr(rdma_algo_token_count),
        _ptr(recv_x), _ptr(recv_x_scales), _ptr(recv_src_idx), _ptr(recv_topk_idx), _ptr(recv_topk_w),
        _ptr(token_rank_slot), _ptr(rank_offset), ws.ptr, ws.nbytes, _stream(stream)), "ep_dispatch_ranks_with_layout")


def ep_expert_reduce_ranks(shape, recv_x, recv_x_scales, rank_offset, recv_topk_idx, recv_topk_w, factor,
                           partial, stream=None):
    cap, H, k, R = shape.rank_rows_cap, shape.hidden, shape.num_topk, shape.num_ranks
    fp8 = shape.x_format == EP_FMT_FP8_S128
    _need(recv_x, torch.uint8 if fp8 else torch.bfloat16, (cap, H), "recv_x")
    if fp8:
        _need(recv_x_scales, torch.float32, (cap, H // 128), "recv_x_scales")
    _need(rank_offset, torch.int32, (R + 1,), "rank_offset")
    _need(recv_topk_idx, torch.int32, (cap, k), "recv_topk_idx")
    _need(recv_topk_w, torch.float32, (cap, k), "recv_topk_w")
    if factor is not None:
        _need(factor, torch.float32, (shape.num_experts,), "factor")
    _need(partial, torch.bfloat16, (cap, H), "partial")
    _ok(load().ep_expert_reduce_ranks(ctypes.byref(shape), _ptr(recv_x), _ptr(recv_x_scales), _ptr(rank_offset),
                                      _ptr(recv_topk_idx), _ptr(recv_topk_w), _ptr(factor), _ptr(partial),
                                      _stream(stream)), "ep_expert_reduce_ranks")


def ep_combine_ranks(shape, partial, token_rank_slot, y, stream=None):
    T, H, R = shape.num_tokens, shape.hidden, shape.num_ranks
    _need(partial, torch.bfloat16, (shape.rank_rows_cap, H), "partial")
    _need(token_rank_slot, torch.int32, (T, R), "token_rank_slot")
    _need(y, torch.bfloat16, (T, H), "y")
    _ok(load().ep_combine_ranks(ctypes.byref(shape), _ptr(partial), _ptr(token_rank_slot), _ptr(y),
                                _stream(stream)), "ep_combine_ranks")


def ep_quant_fp8_s128(x, q, scales, stream=None):
    rows, H = x.shape
    _need(x, torch.bfloat16, (rows, H), "x")
    _need(q, torch.uint8, (rows, H), "q")
    _need(scales, torch.float32, (rows, H // 128), "scales")
    _ok(load().ep_quant_fp8_s128(rows, H, _ptr(x), _ptr(q), _ptr(scales), _stream(stream)),
        "ep_quant_fp8_s128")


def ep_expert_scale_bf16(shape, expert_offset, factor, recv, out, stream=None):
    _ok(load().ep_expert_scale_bf16(ctypes.byref(shape), _ptr(expert_offset), _ptr(factor), _ptr(recv),
                                    _ptr(out), _stream(stream)), "ep_expert_scale_bf16")


def ep_expert_requant_mxfp8(shape, expert_offset, factor, recv_q, recv_scales, out_q, out_e8m0,
                            stream=None):
    _ok(load().ep_expert_requant_mxfp8(ctypes.byref(shape), _ptr(expert_offset), _ptr(factor),
                                       _ptr(recv_q), _ptr(recv_scales), _ptr(out_q), _ptr(out_e8m0),
                                       _stream(stream)), "ep_expert_requant_mxfp8")


def ep_expert_requant_nvfp4(shape, expert_offset, factor, recv, out_q, out_scales, stream=None):
    _ok(load().ep_expert_requant_nvfp4(ctypes.byref(shape), _ptr(expert_offset), _ptr(factor), _ptr(recv),
                                       _ptr(out_q), _ptr(out_scales), _stream(stream)),
        "ep_expert_requant_nvfp4")


def ep_accounting(shape, own_node, num_tokens_per_rank, num_tokens_per_node, rdma_algo_token_count,
                  valid_pairs) -> dict:
    """Host arithmetic on host copies of the counts (numpy int32 arrays)."""
    import numpy as np
    r = np.ascontiguousarray(num_tokens_per_rank, np.int32)
    n = np.ascontiguousarray(num_tokens_per_node, np.int32)
    out = ep_accounting_t()
    _ok(load().ep_accounting(ctypes.byref(shape), int(own_node), r.ctypes.data_as(ctypes.c_void_p),
                             n.ctypes.data_as(ctypes.c_void_p), int(rdma_algo_token_count),
                             int(valid_pairs), ctypes.byref(out)), "ep_accounting")
    return out.as_dict()


def ep_calib_copy(src, dst, nbytes, stream=None):
    _ok(load().ep_calib_copy(_ptr(src), _ptr(dst), int(nbytes), _stream(stream)), "ep_calib_copy")


EP_STREAM_READ, EP_STREAM_READ_NT, EP_STREAM_WRITE, EP_STREAM_WRITE_NT, EP_STREAM_COPY, EP_STREAM_COPY_NT = range(6)


def ep_stream(kind, src, dst, nbytes, chunk_bytes, waves, stream=None):
    """Streaming measurement kernel (read / write / copy, plain or non-temporal)."""
    for t in (src, dst):
        if t is not None and t.numel() * t.element_size() < (16 if t is dst and kind < 2 else nbytes):
            raise ValueError("ep_stream: buffer smaller than the bytes streamed")
    _ok(load().ep_stream(int(kind), _ptr(src), _ptr(dst), int(nbytes), int(chunk_bytes), int(waves),
                         _stream(stream)), "ep_stream")


# --------------------------------------------------------------------------- allocating forms

@dataclass
class Handle:
    """What combine needs from dispatch: the receiver-side layout."""
    shape: ep_shape
    token_slot: torch.Tensor      # [T, k] int32
    expert_offset: torch.Tensor   # [E + 1] int32
    topk_w: torch.Tensor          # [T, k] fp32


def dispatch_layout(topk_idx, shape, ws: Workspace, stream=None) -> dict:
    dev = topk_idx.device
    T, R, E, N = shape.num_tokens, shape.num_ranks, shape.num_experts, shape.num_nodes
    out = dict(
        num_tokens_per_rank=torch.empty(R, dtype=torch.int32, device=dev),
        num_tokens_per_expert=torch.empty(E, dtype=torch.int32, device=dev),
        is_token_in_rank=torch.empty((T, R), dtype=torch.uint8, device=dev),
        num_tokens_per_node=torch.empty(N, dtype=torch.int32, device=dev),
        rdma_algo_token_count=torch.empty(1, dtype=torch.int64, device=dev),
    )
    ep_dispatch_layout(shape, topk_idx, out["num_tokens_per_rank"], out["num_tokens_per_expert"],
                       out["is_token_in_rank"], out["num_tokens_per_node"], out["rdma_algo_token_count"],
                       ws, stream)
    return out


def dispatch(x, topk_idx, topk_w, shape, ws: Workspace, x_scales=None, stream=None, from_layout=False):
    """Returns recv_x, recv_x_scales (None for bf16), recv_src_idx, recv_topk_w, handle."""
    dev = x.device
    T, k, H, E = shape.num_tokens, shape.num_topk, shape.hidden, shape.num_experts
    fp8 = shape.x_format == EP_FMT_FP8_S128
    rows = shape.rows
    recv_x = torch.empty((rows, H), dtype=x.dtype, device=dev)
    recv_x_scales = torch.empty((rows, H // 128), dtype=torch.float32, device=dev) if fp8 else None
    recv_src_idx = torch.empty(rows, dtype=torch.int32, device=dev)
    recv_topk_w = torch.empty(rows, dtype=torch.float32, device=dev)
    token_slot = torch.empty((T, k), dtype=torch.int32, device=dev)
    expert_offset = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ep_dispatch(shape, x, x_scales, topk_idx, topk_w, recv_x, recv_x_scales, recv_src_idx, recv_topk_w,
                token_slot, expert_offset, ws, stream, from_layout)
    return recv_x, recv_x_scales, recv_src_idx, recv_topk_w, Handle(shape, token_slot, expert_offset, topk_w)


def dispatch_with_layout(x, topk_idx, topk_w, shape, ws: Workspace, x_scales=None, stream=None):
    """Returns the layout dict and recv_x, recv_x_scales, recv_src_idx, recv_topk_w, handle."""
    dev = x.device
    T, k, H, E, R, N = (shape.num_tokens, shape.num_topk, shape.hidden, shape.num_experts, shape.num_ranks,
                        shape.num_nodes)
    rows = shape.rows
    fp8 = shape.x_format == EP_FMT_FP8_S128
    lay = dict(
        num_tokens_per_rank=torch.empty(R, dtype=torch.int32, device=dev),
        num_tokens_per_expert=torch.empty(E, dtype=torch.int32, device=dev),
        is_token_in_rank=torch.empty((T, R), dtype=torch.uint8, device=dev),
        num_tokens_per_node=torch.empty(N, dtype=torch.int32, device=dev),
        rdma_algo_token_count=torch.empty(1, dtype=torch.int64, device=dev),
    )
    recv_x = torch.empty((rows, H), dtype=x.dtype, device=dev)
    recv_x_scales = torch.empty((rows, H // 128), dtype=torch.float32, device=dev) if fp8 else None
    recv_src_idx = torch.empty(rows, dtype=torch.int32, device=dev)
    recv_topk_w = torch.empty(rows, dtype=torch.float32, device=dev)
    token_slot = torch.empty((T, k), dtype=torch.int32, device=dev)
    expert_offset = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ep_dispatch_with_layout(shape, x, x_scales, topk_idx, topk_w, lay["num_tokens_per_rank"],
                            lay["num_tokens_per_expert"], lay["is_token_in_rank"], lay["num_tokens_per_node"],
                            lay["rdma_algo_token_count"], recv_x, recv_x_scales, recv_src_idx, recv_topk_w,
                            token_slot, expert_offset, ws, stream)
    return lay, recv_x, recv_x_scales, recv_src_idx, recv_topk_w, Handle(shape, token_slot, expert_offset, topk_w)


def combine(expert_out, handle: Handle, expert_out_scales=None, stream=None):
    sh = handle.shape
    y = torch.empty((sh.num_tokens, sh.hidden), dtype=torch.bfloat16, device=expert_out.device)
    ep_combine(sh, expert_out, expert_out_scales, handle.token_slot, handle.topk_w, y, stream)
    return y


def quant_fp8_s128(x, stream=None):
    rows, H = x.shape
    q = torch.empty((rows, H), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, H // 128), dtype=torch.float32, device=x.device)
    ep_quant_fp8_s128(x, q, s, stream)
    return q, s


@dataclass
class RankHandle:
    """What the (token, rank) combine needs from dispatch."""
    shape: ep_shape
    token_rank_slot: torch.Tensor   # [T, R] int32
    rank_offset: torch.Tensor       # [R + 1] int32


def dispatch_ranks(x, topk_idx, topk_w, shape, ws: Workspace, x_scales=None, stream=None) -> dict:
    """(token, rank) dispatch after dispatch_layout on `ws`; returns recv_x,
    recv_x_scales (None for bf16), recv_src_idx, recv_topk_idx, recv_topk_w
    and the handle."""
    dev = x.device
    T, k, H, R = shape.num_tokens, shape.num_topk, shape.hidden, shape.num_ranks
    cap = shape.rank_rows_cap
    fp8 = shape.x_format == EP_FMT_FP8_S128
    out = dict(
        recv_x=torch.empty((cap, H), dtype=x.dtype, device=dev),
        recv_x_scales=torch.empty((cap, H // 128), dtype=torch.float32, device=dev) if fp8 else None,
        recv_src_idx=torch.empty(cap, dtype=torch.int32, device=dev),
        recv_topk_idx=torch.empty((cap, k), dtype=torch.int32, device=dev),
        recv_topk_w=torch.empty((cap, k), dtype=torch.float32, device=dev),
    )
    h = RankHandle(shape, torch.empty((T, R), dtype=torch.int32, device=dev),
                   torch.empty(R + 1, dtype=torch.int32, device=dev))
    ep_dispatch_ranks(shape, x, x_scales, topk_idx, topk_w, out["recv_x"], out["recv_x_scales"],
                      out["recv_src_idx"], out["recv_topk_idx"], out["recv_topk_w"], h.token_rank_slot,
                      h.rank_offset, ws, stream)
    out["handle"] = h
    return out


def dispatch_ranks_with_layout(x, topk_idx, topk_w, shape, ws: Workspace, x_scales=None, stream=None):
    """Layout and (token, rank) dispatch in one call; returns (layout dict, dispatch_ranks-style dict)."""
    dev = x.device
    T, k, H, E, R, N = (shape.num_tokens, shape.num_topk, shape.hidden, shape.num_experts, shape.num_ranks,
                        shape.num_nodes)
    cap = shape.rank_rows_cap
    fp8 = shape.x_format == EP_FMT_FP8_S128
    lay = dict(
        num_tokens_per_rank=torch.empty(R, dtype=torch.int32, device=dev),
        num_tokens_per_expert=torch.empty(E, dtype=torch.int32, device=dev),
        is_token_in_rank=torch.empty((T, R), dtype=torch.uint8, device=dev),
        num_tokens_per_node=torch.empty(N, dtype=torch.int32, device=dev),
        rdma_algo_token_count=torch.empty(1, dtype=torch.int64, device=dev),
    )
    out = dict(
        recv_x=torch.empty((cap, H), dtype=x.dtype, device=dev),
        recv_x_scales=torch.empty((cap, H // 128), dtype=torch.float32, device=dev) if fp8 else None,
        recv_src_idx=torch.empty(cap, dtype=torch.int32, device=dev),
        recv_topk_idx=torch.empty((cap, k), dtype=torch.int32, device=dev),
        recv_topk_w=torch.empty((cap, k), dtype=torch.float32, device=dev),
    )
    h = RankHandle(shape, torch.empty((T, R), dtype=torch.int32, device=dev),
                   torch.empty(R + 1, dtype=torch.int32, device=dev))
    ep_dispatch_ranks_with_layout(shape, x, x_scales, topk_idx, topk_w, lay["num_tokens_per_rank"],
                                  lay["num_tokens_per_expert"], lay["is_token_in_rank"], lay["num_tokens_per_node"],
                                  lay["rdma_algo_token_count"], out["recv_x"], out["recv_x_scales"],
                                  out["recv_src_idx"], out["recv_topk_idx"], out["recv_topk_w"], h.token_rank_slot,
                                  h.rank_offset, ws, stream)
    out["handle"] = h
    return lay, out


def expert_reduce_ranks(d: dict, factor=None, stream=None):
    """The workloads' expert stage over the rows of dispatch_ranks' result."""
    h = d["handle"]
    sh = h.shape
    part = torch.empty((sh.rank_rows_cap, sh.hidden), dtype=torch.bfloat16, device=d["recv_x"].device)
    ep_expert_reduce_ranks(sh, d["recv_x"], d["recv_x_scales"], h.rank_offset, d["recv_topk_idx"],
                           d["recv_topk_w"], factor, part, stream)
    return part


def combine_ranks(partial, handle: RankHandle, stream=None):
    sh = handle.shape
    y = torch.empty((sh.num_tokens, sh.hidden), dtype=torch.bfloat16, device=partial.device)
    ep_combine_ranks(sh, partial, handle.token_rank_slot, y, stream)
    return y
