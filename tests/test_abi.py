"""The C ABI on the host (no GPU): the library loads, exports every function
include/ep.h declares, rejects bad arguments before touching the device, and
its host-side accounting agrees with the oracle's."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from combine_dispatch_layout_02_amd import ep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ep.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ep.LIB_PATH):
        pytest.fail("libep_hip.so is not built (run __graft_entry__.build())")
    return ep.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(ep.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_strerror(lib):
    assert lib.ep_abi_version() == 8
    for rc in (0, -1, -2, -3, -4, -5):
        assert ep.strerror(rc)
    assert "unknown" in ep.strerror(-99)


def test_header_constants_match_binding():
    """Status codes, formats and device error flags: the values ep.h defines
    are the ones the binding uses."""
    src = open(os.path.join(ROOT, "include", "ep.h")).read()
    defines = {n: int(v, 0) for n, v in re.findall(r"#define (EP_ERRFLAG_[A-Z_]+)\s+(0x[0-9a-fA-F]+)u", src)}
    enums = {n: int(v) for n, v in re.findall(r"\b(EP_(?:OK|E[A-Z]+|FMT_[A-Z0-9_]+))\s*=\s*(-?\d+)", src)}
    assert len(defines) == 4 and len(enums) >= 10
    for n, v in {**defines, **enums}.items():
        assert getattr(ep, n) == v, n
    assert len(set(defines.values())) == 4 and all(v & (v - 1) == 0 for v in defines.values())


GOOD = dict(T=4096, H=7168, E=256, R=16, N=2, k=8)


@pytest.mark.parametrize("bad", [
    dict(k=0), dict(k=33), dict(T=-1), dict(E=0), dict(E=4097, R=1, N=1), dict(R=65, E=65 * 4, N=1),
    dict(E=250), dict(N=3), dict(N=32, R=16), dict(H=7), dict(H=12), dict(T=2 ** 28, k=8),
    dict(xf=1, H=7168 + 8), dict(yf=2, H=7168 + 64), dict(xf=5), dict(yf=1)])
def test_validate_rejects(lib, bad):
    p = dict(GOOD)
    xf, yf = bad.pop("xf", 0), bad.pop("yf", 0)
    p.update(bad)
    sh = ep.make_shape(p["T"], p["H"], p["E"], p["R"], p["N"], p["k"], xf, yf)
    assert lib.ep_validate_shape(ctypes.byref(sh)) == ep.EP_EINVAL
    n = ctypes.c_size_t()
    assert lib.ep_workspace_bytes(ctypes.byref(sh), ctypes.byref(n)) == ep.EP_EINVAL


def test_rank_capacity_limits(lib):
    sh = ep.make_shape(64, 256, 16, 4, 1, 2, rank_capacity=-1)
    assert lib.ep_validate_shape(ctypes.byref(sh)) == ep.EP_EINVAL
    sh = ep.make_shape(64, 256, 16, 4, 1, 2, rank_capacity=2 ** 29)
    assert lib.ep_validate_shape(ctypes.byref(sh)) == ep.EP_EINVAL
    sh = ep.make_shape(64, 256, 16, 4, 1, 2, rank_capacity=100)
    assert lib.ep_validate_shape(ctypes.byref(sh)) == ep.EP_OK
    assert sh.rows == 400
    fake = ctypes.c_void_p(0x1000)
    # the expert stage handles the compacted layout only
    assert lib.ep_expert_scale_bf16(ctypes.byref(sh), fake, fake, fake, fake, None) == ep.EP_EINVAL


@pytest.mark.parametrize("p", [GOOD, dict(T=0, H=8, E=1, R=1, N=1, k=1), dict(T=64, H=256, E=16, R=4, N=1, k=2),
                               dict(T=8192, H=7168, E=4096, R=64, N=64, k=32)])
def test_validate_accepts_and_sizes_workspace(lib, p):
    sh = ep.make_shape(p["T"], p["H"], p["E"], p["R"], p["N"], p["k"])
    assert lib.ep_validate_shape(ctypes.byref(sh)) == ep.EP_OK
    n = ctypes.c_size_t()
    assert lib.ep_workspace_bytes(ctypes.byref(sh), ctypes.byref(n)) == ep.EP_OK
    # at least: control words, one int per pair, one int per expert
    assert n.value >= 256 + 4 * p["T"] * p["k"] + 4 * p["E"]
    assert n.value % 256 == 0


def test_calls_reject_before_device_work(lib):
    sh = ep.make_shape(**{"T": 64, "H": 256, "E": 16, "R": 4, "N": 1, "k": 2})
    P = ctypes.c_void_p
    fake = P(0x1000)          # never dereferenced: every call below fails host checks first
    odd = P(0x1008)
    # missing workspace
    assert lib.ep_dispatch_layout(ctypes.byref(sh), fake, fake, fake, fake, fake, fake, None, 0, None) \
        == ep.EP_EWORKSPACE
    # misaligned row buffer
    assert lib.ep_dispatch(ctypes.byref(sh), odd, None, fake, fake, fake, None, fake, fake, fake, fake,
                           fake, 1 << 20, None) == ep.EP_EALIGN
    # scales given for bf16 rows
    assert lib.ep_dispatch(ctypes.byref(sh), fake, fake, fake, fake, fake, None, fake, fake, fake, fake,
                           fake, 1 << 20, None) == ep.EP_EINVAL
    # combine: missing pointers, misaligned output, mxfp8 without scales
    assert lib.ep_combine(ctypes.byref(sh), None, None, fake, fake, fake, None) == ep.EP_EINVAL
    assert lib.ep_combine(ctypes.byref(sh), fake, None, fake, fake, odd, None) == ep.EP_EALIGN
    shm = ep.make_shape(64, 256, 16, 4, 1, 2, 0, ep.EP_FMT_MXFP8)
    assert lib.ep_combine(ctypes.byref(shm), fake, None, fake, fake, fake, None) == ep.EP_EINVAL
    assert lib.ep_quant_fp8_s128(4, 100, fake, fake, fake, None) == ep.EP_EINVAL
    assert lib.ep_calib_copy(fake, fake, 17, None) == ep.EP_EINVAL
    assert lib.ep_workspace_init(P(0x1010), 4096, None) == ep.EP_EALIGN


@pytest.mark.parametrize("name", ["tiny", "prefill2n", "quant"])
def test_accounting_matches_oracle(lib, name):
    from combine_dispatch_layout_02_amd import workloads as W
    inp = W.make_inputs(name, T=512)
    lay = oracle.layout(inp["topk_idx"], inp["E"], inp["R"], inp["N"])
    xf = ep.EP_FMT_FP8_S128 if inp["x_fmt"] == "fp8" else ep.EP_FMT_BF16
    sh = ep.make_shape(inp["T"], inp["H"], inp["E"], inp["R"], inp["N"], inp["k"], xf)
    for own in range(inp["N"]):
        got = ep.ep_accounting(sh, own, lay["num_tokens_per_rank"], lay["num_tokens_per_node"],
                               lay["rdma_algo_token_count"], int(lay["num_tokens_per_expert"].sum()))
        ref = oracle.accounting(inp["H"], inp["R"], inp["N"], own, lay["num_tokens_per_rank"],
                                lay["num_tokens_per_node"], lay["rdma_algo_token_count"])
        for key, val in ref.items():
            assert got[key] == val, key
    T, H, k = inp["T"], inp["H"], inp["k"]
    row = 2 * H if xf == 0 else H + 4 * H // 128
    assert got["hbm_dispatch_bytes"] == T * row + T * k * row + T * k * 16 + T * k * 8 + 4 * (inp["E"] + 1)
    assert got["hbm_combine_bytes"] == T * k * 2 * H + T * 2 * H + T * k * 8


def test_rank_rows_calls_reject_before_device_work(lib):
    P = ctypes.c_void_p
    fake, odd = P(0x1000), P(0x1008)
    sh0 = ep.make_shape(64, 256, 16, 4, 1, 2)                 # rank_rows not set
    sh1 = ep.make_shape(64, 256, 16, 4, 1, 2, rank_rows=1)
    assert lib.ep_validate_shape(ctypes.byref(ep.make_shape(64, 256, 16, 4, 1, 2, rank_rows=2))) == ep.EP_EINVAL
    assert lib.ep_validate_shape(ctypes.byref(ep.make_shape(2 ** 26, 256, 64, 64, 1, 2, rank_rows=1))) \
        == ep.EP_EINVAL                                        # T * R >= 2^31
    assert sh1.rank_rows_cap == 64 * 2
    n0, n1 = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.ep_workspace_bytes(ctypes.byref(sh0), ctypes.byref(n0)) == ep.EP_OK
    assert lib.ep_workspace_bytes(ctypes.byref(sh1), ctypes.byref(n1)) == ep.EP_OK
    # the rank masks: one tile of 512 tokens (16 waves of 64 pairs at top-2),
    # 4 ranks, 8 words of 64 tokens each
    assert n1.value >= n0.value + 1 * 4 * 8 * 8
    assert lib.ep_dispatch_ranks(ctypes.byref(sh0), fake, None, fake, fake, fake, None, *([fake] * 5),
                                 fake, 1 << 20, None) == ep.EP_EINVAL
    assert lib.ep_dispatch_ranks(ctypes.byref(sh1), odd, None, fake, fake, fake, None, *([fake] * 5),
                                 fake, 1 << 20, None) == ep.EP_EALIGN
    assert lib.ep_dispatch_ranks(ctypes.byref(sh1), fake, fake, fake, fake, fake, None, *([fake] * 5),
                                 fake, 1 << 20, None) == ep.EP_EINVAL   # scales for bf16 rows
    assert lib.ep_dispatch_ranks(ctypes.byref(sh1), fake, None, fake, fake, fake, None, *([fake] * 5),
                                 fake, 16, None) == ep.EP_EWORKSPACE
    assert lib.ep_expert_reduce_ranks(ctypes.byref(sh0), fake, None, fake, fake, fake, None, fake, None) \
        == ep.EP_EINVAL
    assert lib.ep_expert_reduce_ranks(ctypes.byref(sh1), fake, fake, fake, fake, fake, None, fake, None) \
        == ep.EP_EINVAL                                        # scales for bf16 rows
    assert lib.ep_expert_reduce_ranks(ctypes.byref(sh1), fake, None, fake, fake, fake, None, odd, None) \
        == ep.EP_EALIGN
    shm = ep.make_shape(64, 256, 16, 4, 1, 2, 0, ep.EP_FMT_MXFP8, rank_rows=1)
    assert lib.ep_combine_ranks(ctypes.byref(shm), fake, fake, fake, None) == ep.EP_EINVAL
    assert lib.ep_combine_ranks(ctypes.byref(sh0), fake, fake, fake, None) == ep.EP_EINVAL
    assert lib.ep_combine_ranks(ctypes.byref(sh1), fake, fake, odd, None) == ep.EP_EALIGN
    assert lib.ep_combine_ranks(ctypes.byref(sh1), None, fake, fake, None) == ep.EP_EINVAL


@pytest.mark.parametrize("name", ["tiny", "prefill2n", "quant"])
def test_rank_rows_accounting(lib, name):
    from combine_dispatch_layout_02_amd import workloads as W
    inp = W.make_inputs(name, T=512)
    lay = oracle.layout(inp["topk_idx"], inp["E"], inp["R"], inp["N"])
    sr = oracle.slots_ranks(inp["topk_idx"], inp["topk_w"], inp["E"], inp["R"])
    xf = ep.EP_FMT_FP8_S128 if inp["x_fmt"] == "fp8" else ep.EP_FMT_BF16
    sh = ep.make_shape(inp["T"], inp["H"], inp["E"], inp["R"], inp["N"], inp["k"], xf, rank_rows=1)
    got = ep.ep_accounting(sh, 0, lay["num_tokens_per_rank"], lay["num_tokens_per_node"],
                           lay["rdma_algo_token_count"], int(lay["num_tokens_per_expert"].sum()))
    T, H, k, R = inp["T"], inp["H"], inp["k"], inp["R"]
    rows = int(sr["rank_offset"][-1])          # the oracle's row count
    row = 2 * H if xf == 0 else H + 4 * H // 128
    assert got["nvl_tokens"] == rows
    assert got["hbm_dispatch_ranks_bytes"] == (T * row + rows * row + T * k * 12 + T * R * 4
                                               + rows * (4 + 8 * k) + 4 * (R + 1))
    assert got["hbm_combine_ranks_bytes"] == rows * 2 * H + T * 2 * H + T * R * 4


def test_dispatch_with_layout_rejects_before_device_work(lib):
    P = ctypes.c_void_p
    fake, odd = P(0x1000), P(0x1008)
    sh = ep.make_shape(64, 256, 16, 4, 1, 2)
    f = [fake] * 5   # layout outputs

    def call(x=fake, xs=None, lay=f, recv=fake, rs=None, ws=fake, nbytes=1 << 20):
        return lib.ep_dispatch_with_layout(ctypes.byref(sh), x, xs, fake, fake, *lay, recv, rs, fake, fake, fake,
                                           fake, ws, nbytes, None)
    assert call(x=odd) == ep.EP_EALIGN
    assert call(xs=fake) == ep.EP_EINVAL                          # scales for bf16 rows
    assert call(lay=[None] + f[1:]) == ep.EP_EINVAL               # a layout output missing
    assert call(lay=f[:2] + [odd] + f[3:]) == ep.EP_EALIGN        # token-in-rank map misaligned (R % 4 == 0)
    assert call(ws=None) == ep.EP_EWORKSPACE
    assert call(nbytes=16) == ep.EP_EWORKSPACE


def test_cached_dispatch_rejects_before_device_work(lib):
    P = ctypes.c_void_p
    fake, odd = P(0x1000), P(0x1008)
    sh = ep.make_shape(64, 256, 16, 4, 1, 2)
    shr = ep.make_shape(64, 256, 16, 4, 1, 2, rank_rows=1)
    shq = ep.make_shape(64, 256, 16, 4, 1, 2, ep.EP_FMT_FP8_S128)
    assert lib.ep_dispatch_cached(ctypes.byref(sh), odd, None, fake, fake, None, None) == ep.EP_EALIGN
    assert lib.ep_dispatch_cached(ctypes.byref(sh), fake, fake, fake, fake, None, None) == ep.EP_EINVAL
    assert lib.ep_dispatch_cached(ctypes.byref(shq), fake, fake, fake, fake, None, None) == ep.EP_EINVAL
    assert lib.ep_dispatch_cached(ctypes.byref(sh), fake, None, None, fake, None, None) == ep.EP_EINVAL
    assert lib.ep_dispatch_ranks_cached(ctypes.byref(sh), fake, None, fake, fake, None, None) == ep.EP_EINVAL
    assert lib.ep_dispatch_ranks_cached(ctypes.byref(shr), fake, None, fake, odd, None, None) == ep.EP_EALIGN
    empty = ep.make_shape(0, 256, 16, 4, 1, 2)
    assert lib.ep_dispatch_cached(ctypes.byref(empty), None, None, None, None, None, None) == ep.EP_OK
