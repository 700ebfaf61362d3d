"""Pins of the oracle's slot assignment and dispatch copy (CPU only).

The slot order is the token-major compacted layout (MSCCL++ PR 860,
RANK_MAJOR commit: the default places tokens at compacted prefix offsets):
expert segments back to back in expert order, pairs in (t, j) order inside
a segment.  Pinned by a brute-force lexicographic sort of (expert, t, j)
triples, by the bijection / stability invariants, and by an exhaustive
micro-case.
"""
import itertools

import numpy as np
import pytest

import oracle
from combine_dispatch_layout_02_amd import workloads as W


def _brute_slots(idx, E):
    T, k = idx.shape
    triples = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k) if 0 <= idx[t, j] < E)
    slot = -np.ones((T, k), np.int64)
    for pos, (_, t, j) in enumerate(triples):
        slot[t, j] = pos
    return slot


def _check_invariants(idx, w, E, sl):
    T, k = idx.shape
    ts, off, src, rw = sl["token_slot"], sl["expert_offset"], sl["recv_src_idx"], sl["recv_topk_w"]
    valid = (idx >= 0) & (idx < E)
    V = int(valid.sum())
    assert off[0] == 0 and off[E] == V
    assert (np.diff(off) >= 0).all()
    assert (ts[~valid] == -1).all()
    got = np.sort(ts[valid])
    np.testing.assert_array_equal(got, np.arange(V))          # bijection onto [0, V)
    tt, jj = np.nonzero(valid)
    np.testing.assert_array_equal(src[ts[tt, jj]], tt)         # source index map
    np.testing.assert_array_equal(rw[ts[tt, jj]].view(np.uint32), w[tt, jj].view(np.uint32))
    for e in range(E):                                          # segment = expert's pairs
        seg = np.arange(off[e], off[e + 1])
        assert (idx[tt[np.isin(ts[tt, jj], seg)], jj[np.isin(ts[tt, jj], seg)]] == e).all()
        assert len(seg) == int((idx == e).sum())
        assert (np.diff(src[seg]) >= 0).all()                   # stable: ascending t


@pytest.mark.parametrize("replace,mask", [(False, 0.0), (True, 0.0), (False, 0.3), (True, 0.25)])
def test_brute_force_small(replace, mask):
    rng = np.random.default_rng(11)
    E, k, T = 12, 4, 50
    idx = (rng.integers(0, E, (T, k)) if replace else np.argsort(rng.random((T, E)), 1)[:, :k]).astype(np.int64)
    idx[rng.random((T, k)) < mask] = -1
    idx[0, 0] = E + 3  # an invalid id is treated as masked
    w = rng.random((T, k), dtype=np.float32)
    sl = oracle.slots(idx, w, E)
    np.testing.assert_array_equal(sl["token_slot"], _brute_slots(idx, E))
    _check_invariants(idx, w, E, sl)


def test_exhaustive_pairs():
    E = 8
    idx = np.array(list(itertools.combinations(range(E), 2)), np.int64)
    idx = np.concatenate([idx, idx[:, ::-1]])  # both slot orders of every pair
    w = np.ones(idx.shape, np.float32)
    sl = oracle.slots(idx, w, E)
    np.testing.assert_array_equal(sl["token_slot"], _brute_slots(idx, E))
    # every expert appears in 7 pairs, twice over
    assert np.diff(sl["expert_offset"]).tolist() == [14] * E


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_invariants_on_workloads(name):
    inp = W.make_inputs(name, T=min(W.WORKLOADS[name]["T"], 1024))
    sl = oracle.slots(inp["topk_idx"], inp["topk_w"], inp["E"])
    _check_invariants(inp["topk_idx"], inp["topk_w"], inp["E"], sl)
    if name == "tiny":
        np.testing.assert_array_equal(sl["token_slot"], _brute_slots(inp["topk_idx"], inp["E"]))


def test_dispatch_rows_bitwise():
    inp = W.make_inputs("tiny", mask_frac=0.2)
    sl = oracle.slots(inp["topk_idx"], inp["topk_w"], inp["E"])
    recv = oracle.dispatch_rows(inp["x"], sl["token_slot"])
    V = sl["expert_offset"][-1]
    for s in range(V):
        np.testing.assert_array_equal(recv[s], inp["x"][sl["recv_src_idx"][s]])
    # scale rows and byte rows move the same way
    scales = np.arange(inp["T"] * 2, dtype=np.float32).reshape(inp["T"], 2)
    rs = oracle.dispatch_rows(scales, sl["token_slot"])
    np.testing.assert_array_equal(rs[:V], scales[sl["recv_src_idx"][:V]])


def _brute_rank_major(idx, E, R, M):
    T, k = idx.shape
    epr = E // R
    slot = -np.ones((T, k), np.int64)
    dropped = 0
    for r in range(R):
        pairs = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k)
                       if r * epr <= idx[t, j] < (r + 1) * epr)
        for pos, (_, t, j) in enumerate(pairs):
            if pos < M:
                slot[t, j] = r * M + pos
            else:
                dropped += 1
    return slot, dropped


@pytest.mark.parametrize("M", [1, 7, 30, 64])
def test_rank_major_brute_force(M):
    """RANK_MAJOR (MSCCL++ PR 860, RANK_MAJOR commit): rank r owns rows
    [r*M, (r+1)*M); inside, expert then (t, j) order; pairs past M dropped."""
    rng = np.random.default_rng(9)
    E, R, k, T = 16, 4, 3, 40
    idx = rng.integers(-1, E, (T, k)).astype(np.int64)
    w = rng.random((T, k), dtype=np.float32)
    rm = oracle.slots_rank_major(idx, w, E, R, M)
    ref, dropped = _brute_rank_major(idx, E, R, M)
    np.testing.assert_array_equal(rm["token_slot"], ref)
    assert rm["dropped"] == dropped
    tt, jj = np.nonzero(ref >= 0)
    np.testing.assert_array_equal(rm["recv_src_idx"][ref[tt, jj]], tt)


def test_rank_major_reduces_bitwise_to_token_major():
    """The page states the combine over RANK_MAJOR slots reduces bit-exactly
    to the token-major result (the combine is layout-agnostic)."""
    inp = W.make_inputs("prefill2n", T=256, H=512, mask_frac=0.1)
    tm = oracle.run_path(inp)
    M = int(max(np.diff(tm["slots"]["expert_offset"][:: inp["E"] // inp["R"]])))
    rm = oracle.run_path(dict(inp, rank_capacity=M))
    assert rm["slots"]["dropped"] == 0
    np.testing.assert_array_equal(rm["y"], tm["y"])
    # same place inside each rank's block
    epr = inp["E"] // inp["R"]
    off = tm["slots"]["expert_offset"]
    ts_tm, ts_rm = tm["slots"]["token_slot"], rm["slots"]["token_slot"]
    r = np.where(inp["topk_idx"] >= 0, inp["topk_idx"] // epr, 0)
    valid = inp["topk_idx"] >= 0
    np.testing.assert_array_equal((ts_rm - r * M)[valid], (ts_tm - off[r * epr])[valid])
