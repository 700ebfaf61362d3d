"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Bar: layout counts, slots, index maps, dispatched rows, fp8 rows / scales and
mxfp8 payloads bit-exact; combine within 1 bf16 ulp per element (the fp32
fma chain in slot order is reproduced exactly, so the tests also report the
count of differing elements, expected 0).  Every workload (the five
configurations and the nvfp4 payload) runs at its full size, in the launch
configuration the benchmark uses, with the plan reused, planned again and
in one call; the RANK_MAJOR layout runs at the prefill shape in both forms.
The edge cases cover ragged, empty and all-masked inputs, masked slots,
duplicate experts, one or two experts, invalid ids, plan-tile counts on both
sides of every path's limits, the shape limits, rows of 64 K elements, and
receive buffers past 2 and 4 GiB.
"""
import numpy as np
import pytest

import oracle
from combine_dispatch_layout_02_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from combine_dispatch_layout_02_amd import ep
    ep.load()  # fails loudly if the HIP library is missing


def _run_both(inp, from_layout=True, with_layout=False):
    import gpu_path
    print(f"case {inp.get('name')} T={inp['T']} H={inp['H']} E={inp['E']} R={inp['R']} N={inp['N']} "
          f"k={inp['k']} seed={inp.get('seed')} from_layout={from_layout} with_layout={with_layout}", flush=True)
    g = gpu_path.run(inp, from_layout=from_layout, with_layout=with_layout)
    r = oracle.run_path(inp)
    ndiff = gpu_path.compare(g, r, inp.get("x_fmt") == "fp8", inp.get("y_fmt") == "nvfp4")
    return g, r, ndiff


@pytest.mark.parametrize("from_layout", [True, False], ids=["from_layout", "standalone"])
@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_full_size(name, from_layout):
    g, r, ndiff = _run_both(W.make_inputs(name), from_layout)
    assert ndiff == 0
    cfg = W.WORKLOADS[name]
    if cfg["x_fmt"] == "bf16" and cfg.get("y_fmt", "bf16") == "bf16" and cfg["expert"] == "identity":
        inp = W.make_inputs(name)
        np.testing.assert_array_equal(g["y"], inp["x"])   # identity round trip


@pytest.mark.parametrize("T", [1, 63, 257, 1000, 1025])
def test_ragged_token_counts(T):
    _, _, ndiff = _run_both(W.make_inputs("decode", T=T, H=1024))
    assert ndiff == 0


@pytest.mark.parametrize("kw", [
    dict(mask_frac=0.3), dict(mask_frac=0.3, mask_tokens=0.1), dict(routing="replace"),
    dict(routing="replace", mask_frac=0.2, k=16), dict(k=1), dict(E=16, R=16, N=16, k=4),
    dict(E=64, R=64, N=8, k=8), dict(E=4096, R=64, N=64, k=32, T=300), dict(H=8, T=100),
    dict(H=7176, T=130),
    dict(T=5000, H=2048, k=6, mask_frac=0.1),    # enough waves for the multi-vector combine, k not 8
    dict(T=13000, H=1024, k=8, mask_frac=0.1)])  # receive rows past the plain-store budget, short rows
def test_edge_cases_bf16(kw):
    kw = dict(kw)
    base = dict(T=kw.pop("T", 700), H=kw.pop("H", 512))
    base.update(kw)
    for from_layout in (True, False):
        _, _, ndiff = _run_both(W.make_inputs("tiny", **base), from_layout)
        assert ndiff == 0


@pytest.mark.parametrize("kw", [dict(mask_frac=0.25), dict(routing="replace", T=333), dict(E=32, R=8, N=2),
                                dict(k=6, T=300, mask_frac=0.1)])
def test_edge_cases_quantized(kw):
    kw = dict(kw)
    base = dict(T=kw.pop("T", 500), H=1024)
    base.update(kw)
    _, _, ndiff = _run_both(W.make_inputs("quant", **base))
    assert ndiff == 0


def test_scaled_expert_with_masks():
    _, _, ndiff = _run_both(W.make_inputs("decode", T=200, mask_frac=0.2))
    assert ndiff == 0


# Wide rows: 64 K elements (128 KB bf16 rows), so every kernel loops over
# several passes per wave and the dispatch and combine run 16 to 64 waves
# per token; bf16 at a hidden size that is no multiple of 128, fp8 rows with
# 512 scales each, and the nvfp4 payload.
@pytest.mark.parametrize("name,T,H", [("tiny", 100, 65536), ("tiny", 300, 65528), ("quant", 100, 65536),
                                      ("quant", 300, 65536), ("nvfp4", 300, 65536)])
def test_wide_rows(name, T, H):
    inp = W.make_inputs(name, T=T, H=H, E=64, R=8, N=2, k=8, mask_frac=0.1)
    forms = [dict(from_layout=True), dict(with_layout=True)]
    if name == "tiny":
        forms.append(dict(from_layout=False))
    for form in forms:
        _, _, ndiff = _run_both(inp, **form)
        assert ndiff == 0


# Every pair on one or two experts: one expert segment holds (nearly) every
# receive row, and every token reaches every rank and node.
@pytest.mark.parametrize("kw", [dict(E=1, R=1, N=1, k=1, T=700),
                                dict(E=2, R=1, N=1, k=4, T=3000, routing="replace"),
                                dict(E=2, R=2, N=2, k=2, T=300)])
def test_one_or_two_experts(kw):
    inp = W.make_inputs("tiny", H=256, **kw)
    for form in (dict(from_layout=True), dict(from_layout=False), dict(with_layout=True)):
        _, _, ndiff = _run_both(inp, **form)
        assert ndiff == 0


# Every slot masked (T > 0): nothing is counted or dispatched and every y row
# is +0.0, through the plan's copy, the standalone dispatch and the one-call
# form (a single launch at T = 100, count + copy at T = 1000).
@pytest.mark.parametrize("T", [100, 1000])
@pytest.mark.parametrize("name", ["prefill2n", "decode", "quant", "nvfp4"])
def test_all_slots_masked(name, T):
    inp = W.make_inputs(name, T=T, H=1024, mask_tokens=1.0)
    assert (inp["topk_idx"] < 0).all()
    forms = [dict(from_layout=True), dict(from_layout=False), dict(with_layout=True)]
    for kw in forms:
        g, _, ndiff = _run_both(inp, **kw)
        assert ndiff == 0
        assert not g["y"].any()
        assert g["layout"]["rdma_algo_token_count"] == 0
        assert (g["slots"]["expert_offset"] == 0).all()
    if name == "prefill2n":   # RANK_MAJOR blocks of one row per rank
        for kw in forms:
            g, _, ndiff = _run_both(dict(inp, rank_capacity=1), **kw)
            assert ndiff == 0
            assert not g["y"].any()


@pytest.mark.parametrize("from_layout", [True, False])
def test_empty_batch(from_layout):
    import gpu_path
    inp = W.make_inputs("tiny", T=0)
    g = gpu_path.run(inp, from_layout=from_layout)
    assert g["layout"]["rdma_algo_token_count"] == 0
    assert (g["layout"]["num_tokens_per_rank"] == 0).all()
    assert (g["layout"]["num_tokens_per_expert"] == 0).all()
    assert (g["slots"]["expert_offset"] == 0).all()


def test_invalid_ids_are_flagged_and_masked():
    import gpu_path
    inp = W.make_inputs("tiny", T=300, H=256)
    inp["topk_idx"] = inp["topk_idx"].copy()
    inp["topk_idx"][5, 0] = inp["E"] + 7
    inp["topk_idx"][200, 1] = inp["E"]
    g = gpu_path.run(inp, check=False)
    with pytest.raises(RuntimeError, match="flagged"):
        g["ws"].check()
    assert g["ws"].check() == 0   # the flag was cleared
    r = oracle.run_path(inp)
    gpu_path.compare(g, r, False)


def test_repeat_calls_are_deterministic():
    import gpu_path
    inp = W.make_inputs("prefill2n", T=1536)
    a = gpu_path.run(inp)
    b = gpu_path.run(inp)
    for key in ("recv_x", "y"):
        np.testing.assert_array_equal(a[key], b[key])
    np.testing.assert_array_equal(a["slots"]["token_slot"], b["slots"]["token_slot"])


def test_workspace_reuse_across_calls():
    """Every layout / standalone dispatch call rewrites the plan in the
    workspace: three rounds on one workspace with different routings, mixing
    both dispatch entry points, all match the oracle."""
    from combine_dispatch_layout_02_amd import ep
    import gpu_path
    inp = W.make_inputs("prefill2n", T=777, H=256)
    shape = ep.make_shape(777, 256, 256, 16, 2, 8)
    ws = ep.Workspace(shape)
    for seed in range(3):
        inp = W.make_inputs("prefill2n", T=777, H=256, seed=seed)
        idx = torch.from_numpy(inp["topk_idx"]).cuda()
        w = torch.from_numpy(inp["topk_w"]).cuda()
        x = gpu_path.to_dev_bf16(inp["x"])
        lay = ep.dispatch_layout(idx, shape, ws)
        recv_x, _, src, rw, h = ep.dispatch(x, idx, w, shape, ws, from_layout=seed % 2 == 0)
        y = ep.combine(recv_x, h)
        ws.check()
        r = oracle.run_path(inp)
        assert int(lay["rdma_algo_token_count"].item()) == r["layout"]["rdma_algo_token_count"]
        np.testing.assert_array_equal(h.token_slot.cpu().numpy(), r["slots"]["token_slot"])
        np.testing.assert_array_equal(gpu_path.bf16_bits(y), r["y"])


def test_from_layout_requires_a_layout_call():
    from combine_dispatch_layout_02_amd import ep
    import gpu_path
    inp = W.make_inputs("tiny")
    shape = ep.make_shape(inp["T"], inp["H"], inp["E"], inp["R"], inp["N"], inp["k"])
    ws = ep.Workspace(shape)
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    w = torch.from_numpy(inp["topk_w"]).cuda()
    x = gpu_path.to_dev_bf16(inp["x"])
    with pytest.raises(RuntimeError, match="preceding ep_dispatch_layout"):
        ep.dispatch(x, idx, w, shape, ws, from_layout=True)


def test_mxfp8_combine_every_code_and_scale():
    """k = 1, w = 1: y = bf16(e4m3(q) * 2^(e8m0 - 127)) for every e4m3 code and
    every e8m0 byte (row r uses scale byte r for all its groups), through
    ep_combine against the oracle."""
    from combine_dispatch_layout_02_amd import ep
    import gpu_path
    T, H, k = 256, 256, 1
    q = np.tile(np.arange(256, dtype=np.uint8), (T, 1))
    e = np.repeat(np.arange(T, dtype=np.uint8)[:, None], H // 32, axis=1)
    e[255] = 254                   # 0xFF is NaN as a scale; the rows cover every finite one
    slot = np.arange(T, dtype=np.int32).reshape(T, 1)
    w = np.ones((T, k), np.float32)
    ref = oracle.combine_mxfp8(q, e, slot, w)
    shape = ep.make_shape(T, H, 1, 1, 1, k, ep.EP_FMT_BF16, ep.EP_FMT_MXFP8)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ep.ep_combine(shape, torch.from_numpy(q).cuda(), torch.from_numpy(e).cuda(),
                  torch.from_numpy(slot).cuda(), torch.from_numpy(w).cuda(), y)
    got = gpu_path.bf16_bits(y)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("slack", [0, 37])
def test_rank_major_full_size(slack):
    """RANK_MAJOR layout at the prefill shape: parity with the oracle, and y
    bit-identical to the compacted layout's y (PR 860: the combine reduces
    bit-exactly to the token-major result)."""
    import gpu_path
    inp = W.make_inputs("prefill2n")
    off = oracle.slots(inp["topk_idx"], inp["topk_w"], inp["E"])["expert_offset"]
    M = int(max(np.diff(off[:: inp["E"] // inp["R"]]))) + slack
    g_tm = gpu_path.run(inp)
    g, r, ndiff = _run_both(dict(inp, rank_capacity=M))
    assert ndiff == 0
    np.testing.assert_array_equal(g["y"], g_tm["y"])


def test_rank_major_overflow_is_flagged_and_dropped():
    import gpu_path
    inp = dict(W.make_inputs("tiny", T=500, H=256), rank_capacity=100)
    g = gpu_path.run(inp, check=False)
    with pytest.raises(RuntimeError, match="flags 0x4"):
        g["ws"].check()
    r = oracle.run_path(inp)
    assert r["slots"]["dropped"] > 0
    gpu_path.compare(g, r, False)


@pytest.mark.parametrize("kw", [dict(), dict(mask_frac=0.25, T=777), dict(routing="replace", T=300),
                                dict(k=5, T=300)])
def test_nvfp4_payload(kw):
    kw = dict(kw)
    base = dict(T=kw.pop("T", 500), H=1024)
    base.update(kw)
    _, _, ndiff = _run_both(W.make_inputs("nvfp4", **base))
    assert ndiff == 0


def test_nvfp4_combine_every_code_and_scale_kind():
    """k = 1, w = 1: y = bf16(e2m1 * scale) for every e2m1 code under scales
    that are powers of two, general bf16 values, tiny and huge, through
    ep_combine against the oracle."""
    from combine_dispatch_layout_02_amd import ep
    import gpu_path
    rng = np.random.default_rng(4)
    T, H, k = 64, 256, 1
    q = np.tile(np.arange(256, dtype=np.uint8), (T, 1))[:, : H // 2]
    sc = rng.integers(0, 0x7F80, (T, H // 16)).astype(np.uint16)   # finite bf16 scales
    sc[0], sc[1], sc[2] = 0x3F80, 0x3FC0, 0x0001
    slot = np.arange(T, dtype=np.int32).reshape(T, 1)
    w = np.ones((T, k), np.float32)
    ref = oracle.combine_nvfp4(q, sc, slot, w)
    shape = ep.make_shape(T, H, 1, 1, 1, k, ep.EP_FMT_BF16, ep.EP_FMT_NVFP4)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ep.ep_combine(shape, torch.from_numpy(q).cuda(), torch.from_numpy(sc.view(np.int16)).cuda(),
                  torch.from_numpy(slot).cuda(), torch.from_numpy(w).cuda(), y)
    np.testing.assert_array_equal(gpu_path.bf16_bits(y), ref)


# single-launch layout + dispatch: batches of at most 2048 (token, slot) pairs
# (16 pair ids per lane up to 1024 pairs, 32 beyond)
@pytest.mark.parametrize("kw", [
    dict(T=1), dict(T=5), dict(T=64), dict(T=127), dict(T=128), dict(T=128, mask_frac=0.3),
    dict(T=128, mask_frac=0.3, mask_tokens=0.2), dict(T=100, routing="replace"), dict(T=32, k=32, E=4096, R=64, N=64),
    dict(T=1024, k=1), dict(T=64, k=16, routing="replace", mask_frac=0.2), dict(T=128, H=8),
    dict(T=129), dict(T=200, mask_frac=0.2), dict(T=256), dict(T=2048, k=1), dict(T=64, k=32, E=4096, R=64, N=64),
    dict(T=256, routing="replace", H=8),
    dict(T=257)])   # 2056 pairs: the multi-launch path through the same call
def test_with_layout_small_batches(kw):
    kw = dict(kw)
    base = dict(H=kw.pop("H", 1024))
    base.update(kw)
    _, _, ndiff = _run_both(W.make_inputs("decode", **base), with_layout=True)
    assert ndiff == 0


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_with_layout_workloads(name):
    """Full size: past 2048 pairs, the count launch and the copy that scans
    the tile counts itself (no scan launch)."""
    _, _, ndiff = _run_both(W.make_inputs(name), with_layout=True)
    assert ndiff == 0


# Layout + dispatch in two launches (count, then the copy that rebuilds the
# segment starts from the tile counts): one lane per tile and a wave sum per
# slot, a second pass past 64 tiles, up to 256 tiles; 257 tiles and more take
# the scan launch.  At E = 256, R = 16, N = 2, top-8 a tile holds 128 tokens.
@pytest.mark.parametrize("tiles", [3, 63, 64, 65, 128, 255, 256, 257])
def test_layout_in_copy_tile_edges(tiles):
    inp = W.make_inputs("tiny", T=tiles * 128 - 3, H=64, E=256, R=16, N=2, k=8, mask_frac=0.05)
    _, _, ndiff = _run_both(inp, with_layout=True)
    assert ndiff == 0


def _rank_capacity(inp, slack=0):
    """The largest rank's pair count (plus slack): no pair is dropped."""
    off = oracle.slots(inp["topk_idx"], inp["topk_w"], inp["E"])["expert_offset"]
    return int(max(np.diff(off[:: inp["E"] // inp["R"]]))) + slack


# RANK_MAJOR through the one-call form: from 2 to 256 plan tiles the copy
# also rebuilds each rank's compacted start from the tile pairs of the
# rank's first expert; 1 tile and 257 tiles take the launches of the plan.
@pytest.mark.parametrize("tiles", [1, 2, 3, 64, 65, 256, 257])
def test_rank_major_with_layout_tile_edges(tiles):
    inp = W.make_inputs("tiny", T=tiles * 128 - 3, H=64, E=256, R=16, N=2, k=8, mask_frac=0.05)
    inp["rank_capacity"] = _rank_capacity(inp, 5)
    _, _, ndiff = _run_both(inp, with_layout=True)
    assert ndiff == 0


@pytest.mark.parametrize("slack", [0, 37])
def test_rank_major_with_layout_full_size(slack):
    """The prefill shape in one call: parity with the oracle, and y equal to
    the compacted layout's y bit for bit."""
    import gpu_path
    inp = W.make_inputs("prefill2n")
    g_tm = gpu_path.run(inp, with_layout=True)
    g, r, ndiff = _run_both(dict(inp, rank_capacity=_rank_capacity(inp, slack)), with_layout=True)
    assert ndiff == 0
    np.testing.assert_array_equal(g["y"], g_tm["y"])


@pytest.mark.parametrize("kw", [dict(T=500, H=256), dict(T=3000, H=64, E=96, R=8, N=2, k=8)])   # 1 tile; 24 tiles, 12 experts per rank
def test_rank_major_with_layout_overflow(kw):
    """Capacity below the largest rank's count: the overflowing pairs are
    dropped and flagged in both the plan's copy and the one-call form."""
    import gpu_path
    inp = W.make_inputs("tiny", **kw)
    inp["rank_capacity"] = _rank_capacity(inp) - 7
    for with_layout in (False, True):
        g = gpu_path.run(inp, check=False, with_layout=with_layout)
        with pytest.raises(RuntimeError, match="flags 0x4"):
            g["ws"].check()
        r = oracle.run_path(inp)
        assert r["slots"]["dropped"] > 0
        assert gpu_path.compare(g, r, False) == 0


@pytest.mark.parametrize("kw", [
    dict(T=300, H=64, E=4096, R=64, N=64, k=8),                 # tiles of 8 tokens (38 tiles)
    dict(T=2049, H=64, E=256, R=8, N=1, k=1),                   # tiles of 1024 tokens
    dict(T=65, H=64, E=256, R=16, N=2, k=32, routing="replace"),   # tiles of 32 tokens, repeated experts
    dict(T=1000, H=256, E=64, R=8, N=4, k=6, mask_frac=0.3, mask_tokens=0.1),
    dict(T=777, H=8, E=16, R=4, N=2, k=2),
    dict(T=3000, H=128, E=96, R=12, N=3, k=8, routing="replace", mask_frac=0.1),   # experts not a power of two
])
def test_layout_in_copy_shapes(kw):
    inp = W.make_inputs("tiny", **kw)
    for with_layout, from_layout in ((True, True), (False, False)):   # layout + dispatch; standalone dispatch
        _, _, ndiff = _run_both(inp, from_layout=from_layout, with_layout=with_layout)
        assert ndiff == 0
    # the same shapes in RANK_MAJOR blocks, through the one-call form
    inp = dict(inp, rank_capacity=_rank_capacity(inp, 3))
    _, _, ndiff = _run_both(inp, with_layout=True)
    assert ndiff == 0


@pytest.mark.parametrize("name", ["quant", "nvfp4"])
def test_layout_in_copy_quantized(name):
    _, _, ndiff = _run_both(W.make_inputs(name, T=1500, H=1024, mask_frac=0.1), with_layout=True)
    assert ndiff == 0


@pytest.mark.parametrize("kw", [dict(T=128), dict(T=100, mask_frac=0.25)])
def test_with_layout_quantized(kw):
    _, _, ndiff = _run_both(W.make_inputs("quant", H=1024, **kw), with_layout=True)
    assert ndiff == 0
    _, _, ndiff = _run_both(W.make_inputs("nvfp4", H=1024, **kw), with_layout=True)
    assert ndiff == 0


@pytest.mark.parametrize("T", [100, 1000])   # one launch; count + copy launches
def test_with_layout_flags_invalid_ids(T):
    import gpu_path
    inp = W.make_inputs("decode", T=T, H=512, mask_frac=0.1)
    bad = inp["topk_idx"].copy()
    bad[7, 3] = inp["E"] + 1
    bad[T - 1, 0] = inp["E"] + 100
    inp["topk_idx"] = bad
    g = gpu_path.run(inp, check=False, with_layout=True)
    with pytest.raises(RuntimeError, match="flags 0x1"):
        g["ws"].check()
    assert gpu_path.compare(g, oracle.run_path(inp), False) == 0


@pytest.mark.parametrize("kw", [dict(T=20000, H=64, E=256, R=16, N=2, k=8),      # 157 plan tiles
                                dict(T=40000, H=8, E=64, R=8, N=2, k=4, mask_frac=0.1),
                                dict(T=3000, H=64, E=4096, R=64, N=8, k=32)])   # tiles of 2 tokens
def test_many_plan_tiles(kw):
    """Batches with more plan tiles than the scan keeps in registers (its
    loop form), and tiny tiles at E = 4096."""
    inp = W.make_inputs("tiny", **kw)
    for from_layout in (True, False):
        _, _, ndiff = _run_both(inp, from_layout)
        assert ndiff == 0
    import gpu_path
    g = gpu_path.run_ranks(inp)
    assert gpu_path.compare_ranks(g, oracle.run_path(dict(inp, rank_rows=True)), False) == 0


# At E = 256, R = 16, N = 2, top-8 a plan tile holds 128 tokens and the scan
# block's 1024 threads split each of the 274 count columns into 3 ranges of
# ceil(tiles / 3) tiles, read in batches of 8 while a range fits 32 tiles.
# The tile counts put the ranges just below and just above each batch edge
# (8, 16, 24 tiles), at the 32-tile limit and one tile past it (the loop form).
@pytest.mark.parametrize("tiles", [3, 24, 25, 48, 49, 72, 73, 96, 97])
def test_scan_batch_edges(tiles):
    inp = W.make_inputs("tiny", T=tiles * 128 - 5, H=64, E=256, R=16, N=2, k=8, mask_frac=0.05)
    _, _, ndiff = _run_both(inp)
    assert ndiff == 0
    import gpu_path
    g = gpu_path.run_ranks(inp)
    assert gpu_path.compare_ranks(g, oracle.run_path(dict(inp, rank_rows=True)), False) == 0


@pytest.mark.parametrize("kw", [dict(), dict(mask_frac=0.2, T=333), dict(x_fmt="fp8", T=300, H=1024),
                                dict(rank_capacity="fit"), dict(T=100)])
def test_cached_dispatch_reuses_a_handle(kw):
    """ep_dispatch_cached with the handle of a first dispatch moves a second
    tensor of the same tokens to the same rows (PR 860: cached dispatch with a
    previous handle): the rows equal the oracle's dispatch of that tensor
    under the handle's slots."""
    from combine_dispatch_layout_02_amd import ep
    import gpu_path
    kw = dict(kw)
    fp8 = kw.pop("x_fmt", "bf16") == "fp8"
    cap = kw.pop("rank_capacity", 0)
    base = dict(T=kw.pop("T", 500), H=kw.pop("H", 512))
    base.update(kw)
    inp = W.make_inputs("prefill2n", **base)
    T, H, E, R, N, k = (inp[n] for n in ("T", "H", "E", "R", "N", "k"))
    if cap == "fit":
        ok = (inp["topk_idx"] >= 0) & (inp["topk_idx"] < E)
        cap = int(np.bincount(inp["topk_idx"][ok] // (E // R), minlength=R).max())
    shape = ep.make_shape(T, H, E, R, N, k, ep.EP_FMT_FP8_S128 if fp8 else ep.EP_FMT_BF16, rank_capacity=cap)
    ws = ep.Workspace(shape)
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    w = torch.from_numpy(inp["topk_w"]).cuda()
    x1 = gpu_path.to_dev_bf16(inp["x"])
    x2_bits = W.f32_to_bf16_bits(np.random.default_rng(77).standard_normal((T, H), dtype=np.float32))
    x2 = gpu_path.to_dev_bf16(x2_bits)
    if fp8:
        x1, s1 = ep.quant_fp8_s128(x1)
        x2, s2 = ep.quant_fp8_s128(x2)
    else:
        s1 = s2 = None
    _, _, _, _, h = ep.dispatch(x1, idx, w, shape, ws, x_scales=s1)
    recv2 = torch.zeros((shape.rows, H), dtype=x2.dtype, device="cuda")
    rs2 = torch.zeros((shape.rows, H // 128), dtype=torch.float32, device="cuda") if fp8 else None
    ep.ep_dispatch_cached(shape, x2, s2, h.token_slot, recv2, rs2)
    ws.check()
    ts = h.token_slot.cpu().numpy()
    used = np.sort(ts[ts >= 0])
    src = x2.cpu().numpy() if fp8 else x2_bits
    ref = oracle.dispatch_rows(src, ts, rows=shape.rows)
    got = recv2.cpu().numpy() if fp8 else gpu_path.bf16_bits(recv2)
    np.testing.assert_array_equal(got[used], ref[used])
    if fp8:
        refs = oracle.dispatch_rows(s2.cpu().numpy(), ts, rows=shape.rows)
        np.testing.assert_array_equal(rs2.cpu().numpy()[used].view(np.uint32), refs[used].view(np.uint32))


@pytest.mark.parametrize("kw", [dict(), dict(x_fmt="fp8", H=1024)])
def test_cached_rank_dispatch_reuses_a_handle(kw):
    from combine_dispatch_layout_02_amd import ep
    import gpu_path
    kw = dict(kw)
    fp8 = kw.pop("x_fmt", "bf16") == "fp8"
    inp = W.make_inputs("prefill2n", T=400, H=kw.pop("H", 512), mask_frac=0.1)
    T, H, E, R, N, k = (inp[n] for n in ("T", "H", "E", "R", "N", "k"))
    shape = ep.make_shape(T, H, E, R, N, k, ep.EP_FMT_FP8_S128 if fp8 else ep.EP_FMT_BF16, rank_rows=1)
    ws = ep.Workspace(shape)
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    w = torch.from_numpy(inp["topk_w"]).cuda()
    x1 = gpu_path.to_dev_bf16(inp["x"])
    x2_bits = W.f32_to_bf16_bits(np.random.default_rng(78).standard_normal((T, H), dtype=np.float32))
    x2 = gpu_path.to_dev_bf16(x2_bits)
    if fp8:
        x1, s1 = ep.quant_fp8_s128(x1)
        x2, s2 = ep.quant_fp8_s128(x2)
    else:
        s1 = s2 = None
    ep.dispatch_layout(idx, shape, ws)
    d = ep.dispatch_ranks(x1, idx, w, shape, ws, x_scales=s1)
    cap = shape.rank_rows_cap
    recv2 = torch.zeros((cap, H), dtype=x2.dtype, device="cuda")
    rs2 = torch.zeros((cap, H // 128), dtype=torch.float32, device="cuda") if fp8 else None
    ep.ep_dispatch_ranks_cached(shape, x2, s2, d["handle"].token_rank_slot, recv2, rs2)
    ws.check()
    trs = d["handle"].token_rank_slot.cpu().numpy()
    np.testing.assert_array_equal(trs, oracle.slots_ranks(inp["topk_idx"], inp["topk_w"], E, R)["token_rank_slot"])
    used = np.sort(trs[trs >= 0])
    src = x2.cpu().numpy() if fp8 else x2_bits
    ref = oracle.dispatch_rows(src, trs, rows=cap)
    got = recv2.cpu().numpy() if fp8 else gpu_path.bf16_bits(recv2)
    np.testing.assert_array_equal(got[used], ref[used])
    if fp8:
        refs = oracle.dispatch_rows(s2.cpu().numpy(), trs, rows=cap)
        np.testing.assert_array_equal(rs2.cpu().numpy()[used].view(np.uint32), refs[used].view(np.uint32))


# Receive buffers past 2^31 and 2^32 bytes, so any 32-bit byte offset would
# show: every count, slot and source index in full; receive rows sampled
# (every ~500th used row and the last 64, which lie past 4 GiB in the
# token-major cases); y of sampled tokens against the oracle run on those
# tokens alone (a token's y depends only on its own row, ids and weights).
@pytest.mark.parametrize("case", ["one_call_256_tiles", "plan_313_tiles", "ranks"])
def test_receive_buffer_past_4_gib(case):
    import gpu_path
    from combine_dispatch_layout_02_amd import ep
    T, H = (40000, 7168) if case == "plan_313_tiles" else (32768, 8704)
    inp = W.make_inputs("prefill2n", T=T, H=H)
    E, R, N, k = inp["E"], inp["R"], inp["N"], inp["k"]
    ranks = case == "ranks"
    shape = ep.make_shape(T, H, E, R, N, k, rank_rows=int(ranks))
    row_bytes = 2 * H
    print(f"case large receive buffer {case} T={T} H={H} rows {shape.rows} x {row_bytes} B", flush=True)
    ws = ep.Workspace(shape)
    x = gpu_path.to_dev_bf16(inp["x"])
    idx = torch.from_numpy(inp["topk_idx"]).cuda()
    w = torch.from_numpy(inp["topk_w"]).cuda()
    if ranks:
        lay, d = ep.dispatch_ranks_with_layout(x, idx, w, shape, ws)
        y = ep.combine_ranks(ep.expert_reduce_ranks(d), d["handle"])
        recv, src = d["recv_x"], d["recv_src_idx"]
        ref = oracle.slots_ranks(inp["topk_idx"], inp["topk_w"], E, R)
        np.testing.assert_array_equal(d["handle"].token_rank_slot.cpu().numpy(), ref["token_rank_slot"])
        np.testing.assert_array_equal(d["handle"].rank_offset.cpu().numpy(), ref["rank_offset"])
        nrows = int(ref["rank_offset"][-1])
    else:
        if case == "one_call_256_tiles":
            lay, recv, _, src, rw, h = ep.dispatch_with_layout(x, idx, w, shape, ws)
        else:
            lay = ep.dispatch_layout(idx, shape, ws)
            recv, _, src, rw, h = ep.dispatch(x, idx, w, shape, ws, from_layout=True)
        y = ep.combine(recv, h)
        ref = oracle.slots(inp["topk_idx"], inp["topk_w"], E)
        np.testing.assert_array_equal(h.token_slot.cpu().numpy(), ref["token_slot"])
        np.testing.assert_array_equal(h.expert_offset.cpu().numpy(), ref["expert_offset"])
        nrows = int(ref["expert_offset"][-1])
        np.testing.assert_array_equal(rw.cpu().numpy()[:nrows].view(np.uint32), ref["recv_topk_w"][:nrows].view(np.uint32))
    assert ws.check() == 0
    assert nrows * row_bytes > (1 << 31) and (ranks or nrows * row_bytes > (1 << 32))
    lr = oracle.layout(inp["topk_idx"], E, R, N)
    for key in ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank", "num_tokens_per_node"):
        np.testing.assert_array_equal(lay[key].cpu().numpy(), lr[key], err_msg=key)
    np.testing.assert_array_equal(src.cpu().numpy()[:nrows], ref["recv_src_idx"][:nrows])
    rows = np.unique(np.concatenate([np.arange(0, nrows, 499), np.arange(nrows - 64, nrows)]))
    got = gpu_path.bf16_bits(recv[torch.from_numpy(rows).cuda()])
    np.testing.assert_array_equal(got, inp["x"][ref["recv_src_idx"][rows]])
    toks = np.unique(np.concatenate([np.arange(0, T, 211), np.arange(T - 16, T)]))
    sub = dict(inp, T=len(toks), x=inp["x"][toks], topk_idx=inp["topk_idx"][toks], topk_w=inp["topk_w"][toks],
               rank_rows=ranks)
    np.testing.assert_array_equal(gpu_path.bf16_bits(y[torch.from_numpy(toks).cuda()]), oracle.run_path(sub)["y"])


# The same for the quantized payloads: fp8 rows (2.3 GB of receive rows and
# as many of mxfp8 expert rows) and bf16 rows with an nvfp4 payload (4.6 GB
# of receive rows), through the one-call dispatch, the expert stage and the
# combine.
@pytest.mark.parametrize("name", ["quant", "nvfp4"])
def test_quantized_receive_buffer_past_2_gib(name):
    import gpu_path
    T = 40000
    inp = W.make_inputs(name, T=T)
    E, H = inp["E"], inp["H"]
    fp8 = name == "quant"
    print(f"case large quantized receive buffer {name} T={T} H={H}", flush=True)
    g = gpu_path.run(inp, with_layout=True)
    ref = oracle.slots(inp["topk_idx"], inp["topk_w"], E)
    np.testing.assert_array_equal(g["slots"]["token_slot"], ref["token_slot"])
    np.testing.assert_array_equal(g["slots"]["expert_offset"], ref["expert_offset"])
    nrows = int(ref["expert_offset"][-1])
    assert nrows * (H if fp8 else 2 * H) > (1 << 31)
    np.testing.assert_array_equal(g["slots"]["recv_src_idx"][:nrows], ref["recv_src_idx"][:nrows])
    rows = np.unique(np.concatenate([np.arange(0, nrows, 499), np.arange(nrows - 64, nrows)]))
    src = ref["recv_src_idx"][rows]
    if fp8:
        q, s = oracle.quant_fp8_s128(inp["x"][src])
        np.testing.assert_array_equal(g["recv_x"][rows], q)
        np.testing.assert_array_equal(g["recv_x_scales"][rows].view(np.uint32), s.view(np.uint32))
    else:
        np.testing.assert_array_equal(g["recv_x"][rows], inp["x"][src])
    toks = np.unique(np.concatenate([np.arange(0, T, 211), np.arange(T - 16, T)]))
    sub = dict(inp, T=len(toks), x=inp["x"][toks], topk_idx=inp["topk_idx"][toks], topk_w=inp["topk_w"][toks])
    np.testing.assert_array_equal(g["y"][toks], oracle.run_path(sub)["y"])
