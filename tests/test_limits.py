"""The library's host-side sizing at the edges of the supported range (CPU).

ep_plan_info reports what the launchers will use -- workspace regions, plan
tiling, dynamic LDS per workgroup -- from the same functions the launchers
call.  These tests walk shapes up to the ABI limits (E = 4096, R = N = 64,
k = 32, T * k up to 2^31 - 1, with and without (token, rank) rows) and check,
with sizes written here from how the kernels index the workspace:
  * every region is 256-byte aligned, the regions do not overlap and all of
    them fit ep_workspace_bytes;
  * each region holds what its kernels address;
  * a plan tile holds whole tokens, one pair per count-kernel thread, at most
    1024 threads, and its pair masks fit the 48 KiB the count kernel budgets;
  * every dynamic LDS request fits 64 KiB (gfx950 allows 160 KiB per
    workgroup; the kernels' static LDS is at most 17 KiB and never adds to a
    dynamic request of more than 26 KiB);
  * the grid sizes fit the launch limits;
and that check_shape rejects every shape one step past a limit.
"""
import ctypes
import itertools

import pytest

from combine_dispatch_layout_02_amd import ep

KIB = 1024
LDS_BUDGET = 64 * KIB
MAX_GRID = 2 ** 31 - 1
SCAN_COPY_MAX_TILES = 256   # the copies rebuild the plan themselves up to this many tiles


def _divisors(n, cap):
    return [d for d in range(1, min(n, cap) + 1) if n % d == 0]


def _shapes():
    for E in (1, 8, 48, 96, 256, 384, 768, 1000, 2048, 3072, 4095, 4096):
        rs = _divisors(E, 64)
        for R in sorted({rs[0], rs[len(rs) // 2], rs[-1]}):
            ns = _divisors(R, R)
            for N in sorted({1, ns[len(ns) // 2], R}):
                for k in (1, 2, 8, 31, 32):
                    tmax = (2 ** 31 - 1) // k
                    for T in (0, 1, 257, 2049, 100_000, tmax):
                        for rank_rows in (0, 1):
                            if rank_rows and T * R >= 2 ** 31:
                                continue
                            yield dict(T=T, H=7168, E=E, R=R, N=N, k=k, rank_rows=rank_rows)


SHAPES = list(_shapes())


@pytest.fixture(scope="module")
def lib():
    return ep.load()


def _shape(d, **kw):
    d = dict(d, **kw)
    return ep.make_shape(d["T"], d["H"], d["E"], d["R"], d["N"], d["k"], d.get("xf", 0), d.get("yf", 0),
                         d.get("M", 0), d.get("rank_rows", 0))


def test_walk_reaches_the_limits():
    assert any(d["E"] == 4096 and d["R"] == 64 and d["N"] == 64 and d["k"] == 32 for d in SHAPES)
    assert any(d["T"] * d["k"] == 2 ** 31 - 1 for d in SHAPES)
    assert any(d["rank_rows"] and d["R"] == 64 for d in SHAPES)
    assert len(SHAPES) > 1000


def test_regions_fit_and_cover_what_the_kernels_address(lib):
    for d in SHAPES:
        sh = _shape(d)
        assert lib.ep_validate_shape(ctypes.byref(sh)) == ep.EP_OK, d
        info = ep.plan_info(sh)
        n = ctypes.c_size_t()
        assert lib.ep_workspace_bytes(ctypes.byref(sh), ctypes.byref(n)) == ep.EP_OK
        total = info["workspace_bytes"]
        assert total == n.value and total % 256 == 0, d
        off, size = info["region_offset"], info["region_bytes"]
        assert off[0] == 0
        for i in range(8):
            assert off[i] % 256 == 0, (d, i)
            end = off[i + 1] if i + 1 < 8 else total
            assert off[i] + size[i] <= end, (d, i)

        T, E, R, N, k, rr = d["T"], d["E"], d["R"], d["N"], d["k"], d["rank_rows"]
        tiles, tt, tw, threads = info["tiles"], info["tile_tokens"], info["tile_waves"], info["count_threads"]
        # tiling: whole tokens per tile, one pair per count thread, masks within 48 KiB
        assert tt >= 1 and tiles >= 1 and tiles * tt >= T, d
        assert T == 0 or (tiles - 1) * tt < T, d
        assert tt * k <= threads == 64 * tw <= 1024, d
        assert threads >= tt, d
        assert tw * E * 8 <= 48 * KIB or tw == 1, d
        assert tiles <= MAX_GRID, d
        # the plan word of a pair, (expert << 16) | local rank, stays a non-negative int32
        assert tt * k <= 1 << 16 and ((E - 1) << 16 | (tt * k - 1)) < 1 << 31, d
        # what the kernels address (4-byte counts, 8-byte masks / pairs)
        ctrl, tile_count, local_rank, plan_offset, rank_mask, rank_start, tile_pairs, rank_pairs = size
        assert ctrl >= 4, d
        assert tile_count >= 4 * tiles * (E + R + N), d
        assert local_rank >= 4 * T * k, d
        assert plan_offset >= 4 * (E + 1), d
        assert rank_start >= 4 * (R + 1), d
        if rr:
            assert rank_mask >= 8 * tiles * R * ((tt + 63) // 64), d
        scan_copy = 2 <= tiles <= SCAN_COPY_MAX_TILES
        if scan_copy and not rr:
            assert tile_pairs >= 8 * E * tiles, d
        if scan_copy and rr:
            assert rank_pairs >= 8 * R * tiles, d


def test_lds_requests_fit_the_workgroup_limit(lib):
    worst = {"count": 0, "single": 0, "scan": 0}
    for d in SHAPES:
        for xf, yf in ((0, 0), (1, 2), (0, 3)):
            if (xf or yf) and d["H"] % 128:
                continue
            info = ep.plan_info(_shape(d, xf=xf, yf=yf))
            assert info["count_lds_bytes"] <= LDS_BUDGET, d
            assert info["single_launch_lds_bytes"] <= LDS_BUDGET, d
            assert info["scan_copy_lds_bytes"] <= LDS_BUDGET, d
            if info["single_launch_lds_bytes"]:
                t = info["single_launch_threads"]
                assert 64 <= t <= 1024 and t % 64 == 0, d
                assert d["T"] * d["k"] <= 2048, d   # the single launch only takes small batches
            worst["count"] = max(worst["count"], info["count_lds_bytes"])
            worst["single"] = max(worst["single"], info["single_launch_lds_bytes"])
            worst["scan"] = max(worst["scan"], info["scan_copy_lds_bytes"])
    # the walk reaches the largest requests the formulas allow
    assert worst["count"] > 48 * KIB and worst["single"] > 16 * KIB and worst["scan"] > 16 * KIB, worst


@pytest.mark.parametrize("field,value", [
    ("T", -1), ("k", 0), ("k", 33), ("E", 0), ("E", 4097), ("R", 0), ("R", 65), ("N", 0),
    ("H", 0), ("H", 4), ("H", 7172),
])
def test_shapes_past_a_limit_are_rejected(lib, field, value):
    d = dict(T=64, H=7168, E=256, R=8, N=2, k=8)
    d[field] = value
    assert lib.ep_validate_shape(ctypes.byref(_shape(d))) == ep.EP_EINVAL


def test_limit_edges(lib):
    ok = lambda **kw: lib.ep_validate_shape(ctypes.byref(_shape(dict(T=64, H=7168, E=256, R=8, N=2, k=8), **kw)))
    assert ok(T=(2 ** 31 - 1) // 8) == ep.EP_OK
    assert ok(T=2 ** 31 // 8) == ep.EP_EINVAL                       # T * k = 2^31
    assert ok(E=4096, R=64, N=64, k=32) == ep.EP_OK
    assert ok(E=4096, R=64, N=3, k=32) == ep.EP_EINVAL             # N does not divide R
    assert ok(E=100, R=8) == ep.EP_EINVAL                           # R does not divide E
    assert ok(xf=1, H=7168 + 8) == ep.EP_EINVAL                     # fp8 rows need H % 128 == 0
    assert ok(yf=3, H=7168 + 64) == ep.EP_EINVAL                    # nvfp4 payload likewise
    assert ok(rank_rows=1, T=2 ** 31 // 64, R=64, E=256, N=2, k=1) == ep.EP_EINVAL   # T * R = 2^31
    assert ok(rank_rows=1, T=2 ** 31 // 64 - 1, R=64, E=256, N=2, k=1) == ep.EP_OK
    assert ok(M=2 ** 31 // 8) == ep.EP_EINVAL                       # R * rank_capacity = 2^31
    assert ok(M=2 ** 31 // 8 - 1) == ep.EP_OK
    assert ok(rank_rows=2) == ep.EP_EINVAL


def test_static_scratch_boundary(lib):
    """ep_dispatch_with_layout_static takes every shape whose workspace fits
    its 16 MiB and rejects the others before any device work."""
    P = ctypes.c_void_p
    fake = P(0x1000)
    for T in (1, 1000, 100_000, 400_000, 500_000, 600_000):
        sh = ep.make_shape(T, 256, 256, 8, 1, 8)
        need = ep.plan_info(sh)["workspace_bytes"]
        if need <= ep.EP_STATIC_SCRATCH_BYTES:
            continue   # accepted: it would launch, so it is not called here (no GPU)
        rc = lib.ep_dispatch_with_layout_static(ctypes.byref(sh), fake, None, fake, fake, *([fake] * 5), fake, None,
                                                fake, fake, fake, fake, None)
        assert rc == ep.EP_EWORKSPACE, T
