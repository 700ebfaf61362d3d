"""CPU oracle for MoE expert-parallel dispatch / combine -- TEST INFRASTRUCTURE.

This package is a checker, not part of the product.  Only ``tests/``, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py``
may import it.  The arithmetic lives in ``ep_oracle.c`` (plain C, built with
``gcc -O2 -ffp-contract=off``); this module only marshals numpy arrays into
it.  It shares no code with the HIP library.

Each wrapper names the page passage its C function follows (pages:
"MORI-EP Benchmark", "MoE-EP Benchmark" README, MSCCL++ pull request 860).

Parity status per function (what pins it, all in ``tests/test_oracle_*.py``):
  layout / algo count       worked example 8166 (MORI "Why ... equivalent",
                            Step 4), three independent dedup formulations,
                            closed-form expectations, brute force
  accounting                the worked example's byte counts and the fp8
                            factor (1 + 4/128) / 2
  slots / dispatch rows     brute-force lexicographic sort, bijection and
                            stability invariants
  RANK_MAJOR slots          brute force per rank; the combine over them equal
                            bit for bit to the token-major one
  (token, rank) slots,      brute force on small cases, regions equal to the
  partials and combine      layout's per-rank counts, one rank reducing to
                            the token-major combine, exact small integers,
                            the two-rounding bound, +0.0 for an empty token
  combine bf16 / mxfp8      identity round trip (y == x), fp64 bound, the
                            slot order that is computed
  combine nvfp4             fp64 bound and exactly representable rows
  formats / quantization    exhaustive e4m3 / e8m0 / e2m1 tables against
                            exact rational arithmetic and brute force, torch's
                            bf16 and fp8 casts, the formats' error on N(0,1)
  expert stage              same format pins (it is a composition of them)
  threads() mode            bytes equal to one thread on every workload

Timing only: inside ``with oracle.threads(n):`` the row-level wrappers
(dispatch rows, combines, expert stages, fp8 input quantisation) split their
rows over n threads -- each thread calls the same C function on a block of
tokens (or of experts), whose rows no other block touches -- so the bytes are
those of one thread (a test checks it).  Correctness tests run with one.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libep_oracle.so")
# EP_ORACLE_LIB: load this build instead, as it is (the CPU suite's
# sanitizer run builds one with address / UB sanitizers)
_LIB_OVERRIDE = os.environ.get("EP_ORACLE_LIB")

_lib = None


def build(force: bool = True) -> str:
    """Compile ep_oracle.c into oracle/libep_oracle.so with gcc."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", _LIB_PATH, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
    return _LIB_PATH


class Accounting(ctypes.Structure):
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
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    sig = {
        "oracle_layout": (i64, [i64, i32, i32, i32, i32, P, P, P, P, P, P]),
        "oracle_unique_rows": (None, [i64, i32, i32, P]),
        "oracle_algo_by_unique": (i64, [i64, i32, i32, i32, P, P]),
        "oracle_algo_by_presence": (i64, [i64, i32, i32, i32, P, P]),
        "oracle_accounting": (None, [i32, i32, i32, i32, P, P, i64, ctypes.POINTER(Accounting)]),
        "oracle_slots": (None, [i64, i32, i32, P, P, P, P, P, P]),
        "oracle_slots_rank_major": (i64, [i64, i32, i32, i32, i32, P, P, P, P, P]),
        "oracle_dispatch_rows": (None, [i64, i32, i64, P, P, P]),
        "oracle_slots_ranks": (None, [i64, i32, i32, i32, P, P, P, P, P, P, P]),
        "oracle_expert_reduce_ranks": (None, [i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P]),
        "oracle_combine_ranks": (None, [i64, i32, i32, P, P, P]),
        "oracle_combine_bf16": (None, [i64, i32, i32, P, P, P, P]),
        "oracle_combine_mxfp8": (None, [i64, i32, i32, P, P, P, P, P]),
        "oracle_combine_bf16_f64": (None, [i64, i32, i32, P, P, P, P]),
        "oracle_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
        "oracle_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "oracle_f32_to_e4m3": (ctypes.c_uint8, [ctypes.c_float]),
        "oracle_e4m3_to_f32": (ctypes.c_float, [ctypes.c_uint8]),
        "oracle_e8m0_to_f32": (ctypes.c_float, [ctypes.c_uint8]),
        "oracle_quant_fp8_s128": (None, [i64, i32, P, P, P]),
        "oracle_quant_mxfp8": (None, [i64, i32, P, P, P]),
        "oracle_expert_scale_bf16": (None, [i32, i32, P, P, P, P]),
        "oracle_f32_to_e2m1": (ctypes.c_uint8, [ctypes.c_float]),
        "oracle_e2m1_to_f32": (ctypes.c_float, [ctypes.c_uint8]),
        "oracle_quant_nvfp4": (None, [i64, i32, P, P, P]),
        "oracle_combine_nvfp4": (None, [i64, i32, i32, P, P, P, P, P]),
        "oracle_expert_requant_nvfp4": (None, [i32, i32, P, P, P, P, P]),
        "oracle_expert_requant_mxfp8": (None, [i32, i32, P, P, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


_THREADS = 1
_POOL: ThreadPoolExecutor | None = None


@contextlib.contextmanager
def threads(n: int):
    """Run the row-level wrappers on `n` threads inside the block (timing)."""
    global _THREADS, _POOL
    old = _THREADS
    _THREADS = max(1, int(n))
    if _THREADS > 1 and (_POOL is None or _POOL._max_workers < _THREADS):
        _POOL = ThreadPoolExecutor(max_workers=_THREADS)
    try:
        yield
    finally:
        _THREADS = old


def _split(n: int, fn) -> None:
    """fn(b0, b1) over [0, n) in _THREADS contiguous blocks (one call when
    single-threaded).  ctypes releases the GIL during each C call."""
    nb = min(_THREADS, n)
    if nb <= 1:
        fn(0, n)
        return
    bounds = [n * i // nb for i in range(nb + 1)]
    list(_POOL.map(lambda i: fn(bounds[i], bounds[i + 1]), range(nb)))


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------- layout

def layout(topk_idx: np.ndarray, E: int, R: int, N: int) -> dict:
    """Set-based layout (MORI page, "Why ... equivalent" Steps 1-3 and the
    reference script's per-rank counts)."""
    lib = _load()
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    out = {
        "num_tokens_per_rank": np.zeros(R, np.int32),
        "num_tokens_per_expert": np.zeros(E, np.int32),
        "is_token_in_rank": np.zeros((T, R), np.uint8),
        "num_tokens_per_node": np.zeros(N, np.int32),
    }
    algo = np.zeros(1, np.int64)
    invalid = lib.oracle_layout(T, k, E, R, N, _p(idx), _p(out["num_tokens_per_rank"]),
                                _p(out["num_tokens_per_expert"]), _p(out["is_token_in_rank"]),
                                _p(out["num_tokens_per_node"]), _p(algo))
    out["rdma_algo_token_count"] = int(algo[0])
    out["invalid_ids"] = int(invalid)
    return out


def unique_rows(ids: np.ndarray, num_slots: int) -> np.ndarray:
    """DeepEP-style per-row unique rewrite (MORI page, Step 2)."""
    lib = _load()
    a = _c(ids, np.int64).copy()
    rows, cols = a.shape
    lib.oracle_unique_rows(rows, cols, num_slots, _p(a))
    return a


def algo_by_unique(topk_idx: np.ndarray, E: int, N: int):
    lib = _load()
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    rows = np.empty((T, k), np.int64)
    algo = lib.oracle_algo_by_unique(T, k, E, N, _p(idx), _p(rows))
    return int(algo), rows


def algo_by_presence(topk_idx: np.ndarray, E: int, N: int):
    lib = _load()
    idx = _c(topk_idx, np.int64)
    T, k = idx.shape
    pres = np.empty((T, N), np.uint8)
    algo = lib.oracle_algo_by_presence(T, k, E, N, _p(idx), _p(pres))
    return int(algo), pres


def accounting(H: int, R: int, N: int, own_node: int, num_tokens_per_rank, num_tokens_per_node,
               rdma_algo_token_count: int) -> dict:
    lib = _load()
    a = Accounting()
    lib.oracle_accounting(H, R, N, own_node, _p(_c(num_tokens_per_rank, np.int32)),
                          _p(_c(num_tokens_per_node, np.int32)), int(rdma_algo_token_count),
                          ctypes.byref(a))
    return a.as_dict()


# --------------------------------------------------------------------------- slots / dispatch

def slots(topk_idx: np.ndarray, topk_w: np.ndarray, E: int) -> dict:
    """Token-major compacted slots (PR 860, RANK_MAJOR commit's TOKEN_MAJOR)."""
    lib = _load()
    idx = _c(topk_idx, np.int64)
    w = _c(topk_w, np.float32)
    T, k = idx.shape
    out = {
        "token_slot": np.empty((T, k), np.int32),
        "expert_offset": np.empty(E + 1, np.int32),
        "recv_src_idx": np.full(T * k, -1, np.int32),
        "recv_topk_w": np.zeros(T * k, np.float32),
    }
    lib.oracle_slots(T, k, E, _p(idx), _p(w), _p(out["token_slot"]), _p(out["expert_offset"]),
                     _p(out["recv_src_idx"]), _p(out["recv_topk_w"]))
    return out


def slots_rank_major(topk_idx: np.ndarray, topk_w: np.ndarray, E: int, R: int, M: int) -> dict:
    """RANK_MAJOR fixed-slot layout (PR 860, RANK_MAJOR commit): rank r owns rows
    [r*M, (r+1)*M); pairs past a rank's capacity are dropped (slot -1)."""
    lib = _load()
    idx = _c(topk_idx, np.int64)
    w = _c(topk_w, np.float32)
    T, k = idx.shape
    out = {
        "token_slot": np.empty((T, k), np.int32),
        "recv_src_idx": np.full(R * M, -1, np.int32),
        "recv_topk_w": np.zeros(R * M, np.float32),
    }
    out["dropped"] = int(lib.oracle_slots_rank_major(T, k, E, R, M, _p(idx), _p(w), _p(out["token_slot"]),
                                                     _p(out["recv_src_idx"]), _p(out["recv_topk_w"])))
    return out


def slots_ranks(topk_idx: np.ndarray, topk_w: np.ndarray, E: int, R: int) -> dict:
    """(token, rank) receive rows: one row per token per rank it reaches,
    regions in rank order, ascending t inside a region; plus each row's
    top-k list as its rank sees it (local ids, -1 / weight 0 elsewhere)."""
    lib = _load()
    idx = _c(topk_idx, np.int64)
    w = _c(topk_w, np.float32)
    T, k = idx.shape
    cap = T * min(k, R)
    out = {
        "token_rank_slot": np.empty((T, R), np.int32),
        "rank_offset": np.empty(R + 1, np.int32),
        "recv_src_idx": np.full(cap, -1, np.int32),
        "recv_topk_idx": np.full((cap, k), -1, np.int32),
        "recv_topk_w": np.zeros((cap, k), np.float32),
    }
    lib.oracle_slots_ranks(T, k, E, R, _p(idx), _p(w), _p(out["token_rank_slot"]), _p(out["rank_offset"]),
                           _p(out["recv_src_idx"]), _p(out["recv_topk_idx"]), _p(out["recv_topk_w"]))
    return out


def expert_reduce_ranks(topk_idx, topk_w, E, R, rank_offset, recv_src_idx, recv=None, factor=None,
                        recv_q=None, recv_scales=None):
    """Per received (token, rank) row: the weighted sum over the token's
    experts on that rank of the expert outputs, one bf16 partial row.  The
    rows are bf16 (`recv`) or e4m3 plus fp32 scales per 128 (`recv_q`,
    `recv_scales`)."""
    lib = _load()
    idx = _c(topk_idx, np.int64)
    w = _c(topk_w, np.float32)
    T, k = idx.shape
    if recv_q is not None:
        q = _c(recv_q, np.uint8)
        sc = _c(recv_scales, np.float32)
        rv = None
        rows, H = q.shape
    else:
        rv = _c(recv, np.uint16)
        q = sc = None
        rows, H = rv.shape
    part = np.zeros((rows, H), np.uint16)
    f = None if factor is None else _c(factor, np.float32)
    lib.oracle_expert_reduce_ranks(T, k, E, R, H, _p(idx), _p(w), _p(f), _p(_c(rank_offset, np.int32)),
                                   _p(_c(recv_src_idx, np.int32)), _p(rv), _p(q), _p(sc), _p(part))
    return part


def combine_ranks(partial: np.ndarray, token_rank_slot: np.ndarray) -> np.ndarray:
    """y[t] = bf16 of the fp32 sum, in rank order, of the token's partials."""
    lib = _load()
    pt = _c(partial, np.uint16)
    ts = _c(token_rank_slot, np.int32)
    T, R = ts.shape
    H = pt.shape[1]
    y = np.empty((T, H), np.uint16)
    _split(T, lambda t0, t1: lib.oracle_combine_ranks(t1 - t0, R, H, _p(pt), _p(ts[t0:t1]), _p(y[t0:t1])))
    return y


def dispatch_rows(src: np.ndarray, token_slot: np.ndarray, fill=0, rows=None) -> np.ndarray:
    """recv[token_slot[t, j]] = src[t] bitwise; capacity `rows` (default T*k) rows."""
    lib = _load()
    src = np.ascontiguousarray(src)
    ts = _c(token_slot, np.int32)
    T, k = ts.shape
    recv = np.full(((T * k) if rows is None else rows,) + src.shape[1:], fill, dtype=src.dtype)
    row_bytes = src.dtype.itemsize * int(np.prod(src.shape[1:], dtype=np.int64))
    _split(T, lambda t0, t1: lib.oracle_dispatch_rows(t1 - t0, k, row_bytes, _p(src[t0:t1]), _p(ts[t0:t1]),
                                                       _p(recv)))
    return recv


# --------------------------------------------------------------------------- combine

def combine_bf16(expert_out: np.ndarray, token_slot: np.ndarray, topk_w: np.ndarray) -> np.ndarray:
    lib = _load()
    eo = _c(expert_out, np.uint16)
    ts = _c(token_slot, np.int32)
    w = _c(topk_w, np.float32)
    T, k = ts.shape
    H = eo.shape[1]
    y = np.empty((T, H), np.uint16)
    _split(T, lambda t0, t1: lib.oracle_combine_bf16(t1 - t0, k, H, _p(eo), _p(ts[t0:t1]), _p(w[t0:t1]),
                                                      _p(y[t0:t1])))
    return y


def combine_mxfp8(expert_q: np.ndarray, expert_e8m0: np.ndarray, token_slot: np.ndarray,
                  topk_w: np.ndarray) -> np.ndarray:
    lib = _load()
    q = _c(expert_q, np.uint8)
    sc = _c(expert_e8m0, np.uint8)
    ts = _c(token_slot, np.int32)
    w = _c(topk_w, np.float32)
    T, k = ts.shape
    H = q.shape[1]
    y = np.empty((T, H), np.uint16)
    _split(T, lambda t0, t1: lib.oracle_combine_mxfp8(t1 - t0, k, H, _p(q), _p(sc), _p(ts[t0:t1]), _p(w[t0:t1]),
                                                       _p(y[t0:t1])))
    return y


def combine_bf16_f64(expert_out: np.ndarray, token_slot: np.ndarray, topk_w: np.ndarray):
    lib = _load()
    eo = _c(expert_out, np.uint16)
    ts = _c(token_slot, np.int32)
    w = _c(topk_w, np.float32)
    T, k = ts.shape
    H = eo.shape[1]
    y = np.empty((T, H), np.float64)
    lib.oracle_combine_bf16_f64(T, k, H, _p(eo), _p(ts), _p(w), _p(y))
    return y


# --------------------------------------------------------------------------- formats

def f32_to_bf16(x) -> np.ndarray:
    lib = _load()
    a = np.asarray(x, np.float32).ravel()
    return np.array([lib.oracle_f32_to_bf16(float(v)) for v in a], np.uint16).reshape(np.shape(x))


def bf16_to_f32(b) -> np.ndarray:
    lib = _load()
    a = np.asarray(b, np.uint16).ravel()
    return np.array([lib.oracle_bf16_to_f32(int(v)) for v in a], np.float32).reshape(np.shape(b))


def f32_to_e4m3(x) -> np.ndarray:
    lib = _load()
    a = np.asarray(x, np.float32).ravel()
    return np.array([lib.oracle_f32_to_e4m3(float(v)) for v in a], np.uint8).reshape(np.shape(x))


def e4m3_to_f32(q) -> np.ndarray:
    lib = _load()
    a = np.asarray(q, np.uint8).ravel()
    return np.array([lib.oracle_e4m3_to_f32(int(v)) for v in a], np.float32).reshape(np.shape(q))


def e8m0_to_f32(e) -> np.ndarray:
    lib = _load()
    a = np.asarray(e, np.uint8).ravel()
    return np.array([lib.oracle_e8m0_to_f32(int(v)) for v in a], np.float32).reshape(np.shape(e))


def quant_fp8_s128(x_bf16: np.ndarray):
    lib = _load()
    x = _c(x_bf16, np.uint16)
    rows, H = x.shape
    q = np.empty((rows, H), np.uint8)
    s = np.empty((rows, H // 128), np.float32)
    _split(rows, lambda r0, r1: lib.oracle_quant_fp8_s128(r1 - r0, H, _p(x[r0:r1]), _p(q[r0:r1]), _p(s[r0:r1])))
    return q, s


def quant_mxfp8(v: np.ndarray):
    lib = _load()
    a = _c(v, np.float32)
    rows, H = a.shape
    q = np.empty((rows, H), np.uint8)
    e = np.empty((rows, H // 32), np.uint8)
    lib.oracle_quant_mxfp8(rows, H, _p(a), _p(q), _p(e))
    return q, e


def f32_to_e2m1(x) -> np.ndarray:
    lib = _load()
    a = np.asarray(x, np.float32).ravel()
    return np.array([lib.oracle_f32_to_e2m1(float(v)) for v in a], np.uint8).reshape(np.shape(x))


def e2m1_to_f32(q) -> np.ndarray:
    lib = _load()
    a = np.asarray(q, np.uint8).ravel()
    return np.array([lib.oracle_e2m1_to_f32(int(v)) for v in a], np.float32).reshape(np.shape(q))


def quant_nvfp4(v: np.ndarray):
    lib = _load()
    a = _c(v, np.float32)
    rows, H = a.shape
    q = np.empty((rows, H // 2), np.uint8)
    s = np.empty((rows, H // 16), np.uint16)
    lib.oracle_quant_nvfp4(rows, H, _p(a), _p(q), _p(s))
    return q, s


def combine_nvfp4(expert_q, expert_scales, token_slot, topk_w) -> np.ndarray:
    lib = _load()
    q = _c(expert_q, np.uint8)
    sc = _c(expert_scales, np.uint16)
    ts = _c(token_slot, np.int32)
    w = _c(topk_w, np.float32)
    T, k = ts.shape
    H = q.shape[1] * 2
    y = np.empty((T, H), np.uint16)
    _split(T, lambda t0, t1: lib.oracle_combine_nvfp4(t1 - t0, k, H, _p(q), _p(sc), _p(ts[t0:t1]), _p(w[t0:t1]),
                                                       _p(y[t0:t1])))
    return y


def expert_requant_nvfp4(recv: np.ndarray, expert_offset: np.ndarray, factor=None):
    lib = _load()
    r = _c(recv, np.uint16)
    off = _c(expert_offset, np.int32)
    f = None if factor is None else _c(factor, np.float32)
    E = off.shape[0] - 1
    rows, H = r.shape
    out_q = np.zeros((rows, H // 2), np.uint8)
    out_s = np.zeros((rows, H // 16), np.uint16)
    _split(E, lambda e0, e1: lib.oracle_expert_requant_nvfp4(e1 - e0, H, _p(off[e0:]),
                                                              None if f is None else _p(f[e0:]), _p(r),
                                                              _p(out_q), _p(out_s)))
    return out_q, out_s


def expert_scale_bf16(recv: np.ndarray, expert_offset: np.ndarray, factor: np.ndarray) -> np.ndarray:
    lib = _load()
    r = _c(recv, np.uint16)
    off = _c(expert_offset, np.int32)
    f = _c(factor, np.float32)
    E = off.shape[0] - 1
    H = r.shape[1]
    out = r.copy()
    _split(E, lambda e0, e1: lib.oracle_expert_scale_bf16(e1 - e0, H, _p(off[e0:]), _p(f[e0:]), _p(r), _p(out)))
    return out


def expert_requant_mxfp8(recv_q: np.ndarray, recv_scales: np.ndarray, expert_offset: np.ndarray,
                         factor: np.ndarray | None = None):
    lib = _load()
    q = _c(recv_q, np.uint8)
    sc = _c(recv_scales, np.float32)
    off = _c(expert_offset, np.int32)
    f = None if factor is None else _c(factor, np.float32)
    E = off.shape[0] - 1
    rows, H = q.shape
    out_q = np.zeros((rows, H), np.uint8)
    out_e = np.zeros((rows, H // 32), np.uint8)
    _split(E, lambda e0, e1: lib.oracle_expert_requant_mxfp8(e1 - e0, H, _p(off[e0:]),
                                                              None if f is None else _p(f[e0:]), _p(q), _p(sc),
                                                              _p(out_q), _p(out_e)))
    return out_q, out_e


def run_path(inputs: dict) -> dict:
    """Whole hot path on the CPU for one workload dict (see the package's
    workloads module): layout, slots, dispatch rows, expert stage, combine."""
    T, H, E, R, N, k = (inputs[n] for n in ("T", "H", "E", "R", "N", "k"))
    idx, w = inputs["topk_idx"], inputs["topk_w"]
    out = {"layout": layout(idx, E, R, N)}
    sl = slots(idx, w, E)
    expert = inputs.get("expert", "identity")
    if inputs.get("rank_rows"):   # (token, rank) receive rows with per-rank partials
        sr = slots_ranks(idx, w, E, R)
        out["slots"] = dict(sl, **sr)
        cap = T * min(k, R)
        fac = inputs.get("expert_factor") if expert == "scale" else None
        trs = sr["token_rank_slot"]
        if inputs.get("x_fmt", "bf16") == "fp8":
            q, s = quant_fp8_s128(inputs["x"])
            out["x_q"], out["x_scales"] = q, s
            rq = dispatch_rows(q, trs, rows=cap)
            rs = dispatch_rows(s, trs, rows=cap)
            out["recv_x"], out["recv_x_scales"] = rq, rs
            part = expert_reduce_ranks(idx, w, E, R, sr["rank_offset"], sr["recv_src_idx"], factor=fac,
                                       recv_q=rq, recv_scales=rs)
        else:
            rx = dispatch_rows(inputs["x"], trs, rows=cap)
            out["recv_x"] = rx
            part = expert_reduce_ranks(idx, w, E, R, sr["rank_offset"], sr["recv_src_idx"], rx, fac)
        out["expert_out"] = part
        out["y"] = combine_ranks(part, trs)
        return out
    M = int(inputs.get("rank_capacity", 0))
    rows = None
    if M > 0:   # RANK_MAJOR: same expert_offset (compacted starts), slots at fixed rank blocks
        rm = slots_rank_major(idx, w, E, R, M)
        sl = dict(sl, token_slot=rm["token_slot"], recv_src_idx=rm["recv_src_idx"],
                  recv_topk_w=rm["recv_topk_w"], dropped=rm["dropped"])
        rows = R * M
    out["slots"] = sl
    ts = sl["token_slot"]
    expert = inputs.get("expert", "identity")
    if inputs.get("x_fmt", "bf16") == "fp8":
        q, s = quant_fp8_s128(inputs["x"])
        out["x_q"], out["x_scales"] = q, s
        rq = dispatch_rows(q, ts, rows=rows)
        rs = dispatch_rows(s, ts, rows=rows)
        out["recv_x"], out["recv_x_scales"] = rq, rs
        eq, ee = expert_requant_mxfp8(rq, rs, sl["expert_offset"], inputs.get("expert_factor"))
        out["expert_q"], out["expert_e8m0"] = eq, ee
        out["y"] = combine_mxfp8(eq, ee, ts, w)
    else:
        rx = dispatch_rows(inputs["x"], ts, rows=rows)
        out["recv_x"] = rx
        if inputs.get("y_fmt") == "nvfp4":
            eq, es = expert_requant_nvfp4(rx, sl["expert_offset"], inputs.get("expert_factor"))
            out["expert_q"], out["expert_scales"] = eq, es
            out["y"] = combine_nvfp4(eq, es, ts, w)
            return out
        if expert == "scale":
            eo = expert_scale_bf16(rx, sl["expert_offset"], inputs["expert_factor"])
        else:
            eo = rx
        out["expert_out"] = eo
        out["y"] = combine_bf16(eo, ts, w)
    return out
