"""Randomised pins of the oracle's integer parts against brute force written
here from the definitions (CPU only, hypothesis-driven shapes).

For random small shapes (E = R * experts-per-rank, R = N * ranks-per-node,
masked and out-of-range ids, duplicates allowed):
  * layout: the per-token rank / node sets, the per-rank / per-node /
    per-expert counts and the algo count, from Python sets (MORI-EP
    Benchmark, "Why DeepEP and Mori RDMA token counts are equivalent");
  * token-major slots: position in the lexicographic sort of (expert, t, j);
  * RANK_MAJOR slots: position inside the rank's block, dropped past M;
  * (token, rank) rows: position in the sort of (rank, t).
"""
import numpy as np
import pytest

import oracle

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402


@st.composite
def routing(draw):
    N = draw(st.integers(1, 4))
    G = draw(st.integers(1, 4))          # ranks per node
    R = N * G
    epr = draw(st.integers(1, 4))
    E = R * epr
    k = draw(st.integers(1, 6))
    T = draw(st.integers(0, 40))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    idx = rng.integers(-2, E + 2, size=(T, k)).astype(np.int64)   # masked and out-of-range ids too
    w = rng.random((T, k), dtype=np.float32)
    M = draw(st.integers(1, max(1, T * k)))
    return dict(T=T, k=k, E=E, R=R, N=N, idx=idx, w=w, M=M)


def _valid(e, E):
    return 0 <= e < E


@settings(max_examples=150, deadline=None)
@given(routing())
def test_layout_against_sets(c):
    T, k, E, R, N, idx = c["T"], c["k"], c["E"], c["R"], c["N"], c["idx"]
    lay = oracle.layout(idx, E, R, N)
    epr, epn = E // R, E // N
    ranks = [{int(e) // epr for e in idx[t] if _valid(e, E)} for t in range(T)]
    nodes = [{int(e) // epn for e in idx[t] if _valid(e, E)} for t in range(T)]
    assert lay["num_tokens_per_rank"].tolist() == [sum(r in s for s in ranks) for r in range(R)]
    assert lay["num_tokens_per_node"].tolist() == [sum(n in s for s in nodes) for n in range(N)]
    assert lay["num_tokens_per_expert"].tolist() == [int((idx == e).sum()) for e in range(E)]
    assert lay["rdma_algo_token_count"] == sum(len(s) for s in nodes)
    for t in range(T):
        assert {r for r in range(R) if lay["is_token_in_rank"][t, r]} == ranks[t]
    assert lay["invalid_ids"] == int((idx >= E).sum())


@settings(max_examples=150, deadline=None)
@given(routing())
def test_slots_against_sorts(c):
    T, k, E, R, idx, w, M = c["T"], c["k"], c["E"], c["R"], c["idx"], c["w"], c["M"]
    epr = E // R
    pairs = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k) if _valid(idx[t, j], E))
    # token-major
    sl = oracle.slots(idx, w, E)
    ref = -np.ones((T, k), np.int64)
    for pos, (_, t, j) in enumerate(pairs):
        ref[t, j] = pos
    np.testing.assert_array_equal(sl["token_slot"], ref)
    # RANK_MAJOR
    rm = oracle.slots_rank_major(idx, w, E, R, M)
    ref_rm = -np.ones((T, k), np.int64)
    fill = [0] * R
    dropped = 0
    for e, t, j in pairs:
        r = e // epr
        if fill[r] < M:
            ref_rm[t, j] = r * M + fill[r]
        else:
            dropped += 1
        fill[r] += 1
    np.testing.assert_array_equal(rm["token_slot"], ref_rm)
    assert rm["dropped"] == dropped
    # (token, rank)
    sr = oracle.slots_ranks(idx, w, E, R)
    tr = sorted({(int(e) // epr, t) for t in range(T) for e in idx[t] if _valid(e, E)})
    ref_tr = -np.ones((T, R), np.int64)
    for pos, (r, t) in enumerate(tr):
        ref_tr[t, r] = pos
    np.testing.assert_array_equal(sr["token_rank_slot"], ref_tr)
    assert sr["rank_offset"][-1] == len(tr)
