"""Pins of the oracle's (token, rank) receive layout (CPU only).

The high-throughput layout gives a token one receive row per destination
rank it reaches (MSCCL++ PR 860: DeepEP's expanded receive layout, one row
per (token, source rank) pair; MORI-EP Benchmark, "NVL / XGMI bandwidth":
one row per token and rank).  The destination applies the top-k weights of
its own experts and returns one partial row; combine sums the partials.

Pinned here by
  * a brute-force sort of the (rank, token) pairs for the slot order, and the
    region sizes against the layout's num_tokens_per_rank (itself pinned by
    the pages' worked example);
  * a brute-force build of each row's local top-k list;
  * the one-rank case, where the path is exactly the token-major combine;
  * an exact closed form (small-integer rows, power-of-two weights: no
    rounding anywhere, so y == x bit for bit);
  * the rounding bound of the arithmetic (one bf16 rounding per partial, one
    per output) against an fp64 evaluation, for bf16 and fp8 rows and scaled
    experts.
"""
import numpy as np
import pytest

import oracle
from combine_dispatch_layout_02_amd import workloads as W


def _brute_rank_slots(idx, E, R):
    T, k = idx.shape
    epr = E // R
    pairs = sorted({(int(e) // epr, t) for t in range(T) for e in idx[t] if 0 <= e < E})
    slot = -np.ones((T, R), np.int64)
    for pos, (r, t) in enumerate(pairs):
        slot[t, r] = pos
    return slot


def _brute_local_lists(idx, w, E, R, slot):
    T, k = idx.shape
    epr = E // R
    rows = T * min(k, R)
    li = -np.ones((rows, k), np.int64)
    lw = np.zeros((rows, k), np.float32)
    for t in range(T):
        for r in range(R):
            s = slot[t, r]
            if s < 0:
                continue
            for j in range(k):
                e = int(idx[t, j])
                if 0 <= e < E and e // epr == r:
                    li[s, j] = e - r * epr
                    lw[s, j] = w[t, j]
    return li, lw


@pytest.mark.parametrize("replace,mask", [(False, 0.0), (True, 0.0), (False, 0.3), (True, 0.25)])
def test_brute_force_small(replace, mask):
    rng = np.random.default_rng(5)
    E, R, k, T = 24, 6, 5, 60
    idx = (rng.integers(0, E, (T, k)) if replace else np.argsort(rng.random((T, E)), 1)[:, :k]).astype(np.int64)
    idx[rng.random((T, k)) < mask] = -1
    idx[1, 2] = E + 5          # invalid ids count as masked
    idx[7, :] = -1             # a token that reaches no rank
    w = rng.random((T, k), dtype=np.float32)
    sr = oracle.slots_ranks(idx, w, E, R)
    ref = _brute_rank_slots(idx, E, R)
    np.testing.assert_array_equal(sr["token_rank_slot"], ref)
    V = int((ref >= 0).sum())
    assert sr["rank_offset"][-1] == V
    tt, rr = np.nonzero(ref >= 0)
    np.testing.assert_array_equal(sr["recv_src_idx"][ref[tt, rr]], tt)
    assert (sr["recv_src_idx"][V:] == -1).all()
    li, lw = _brute_local_lists(idx, w, E, R, ref)
    np.testing.assert_array_equal(sr["recv_topk_idx"][:V], li[:V])
    np.testing.assert_array_equal(sr["recv_topk_w"][:V].view(np.uint32), lw[:V].view(np.uint32))
    assert (sr["token_rank_slot"][7] == -1).all()


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill2n", "skewed"])
def test_regions_match_layout(name):
    """Region r holds num_tokens_per_rank[r] rows, and a token has a row on r
    exactly when is_token_in_rank[t, r]."""
    inp = W.make_inputs(name, T=min(W.WORKLOADS[name]["T"], 512))
    idx, E, R, N = inp["topk_idx"], inp["E"], inp["R"], inp["N"]
    lay = oracle.layout(idx, E, R, N)
    sr = oracle.slots_ranks(idx, inp["topk_w"], E, R)
    np.testing.assert_array_equal(np.diff(sr["rank_offset"]), lay["num_tokens_per_rank"])
    np.testing.assert_array_equal(sr["token_rank_slot"] >= 0, lay["is_token_in_rank"].astype(bool))
    # inside a region: ascending t, and the local lists hold every slot on r
    for r in range(R):
        seg = sr["recv_src_idx"][sr["rank_offset"][r]:sr["rank_offset"][r + 1]]
        assert (np.diff(seg) > 0).all()
    rows = sr["rank_offset"][-1]
    assert int((sr["recv_topk_idx"][:rows] >= 0).sum()) == int((idx >= 0).sum())


def test_one_rank_is_token_major_combine():
    """R = 1: each token has one row holding all its experts; its partial is
    the token-major combine's fma chain, and the sum of one partial is the
    partial itself, so y equals the token-major y bit for bit."""
    inp = W.make_inputs("decode", T=64, H=512, R=1, mask_frac=0.2)
    ht = oracle.run_path(dict(inp, rank_rows=True))
    tm = oracle.run_path(inp)
    np.testing.assert_array_equal(ht["y"], tm["y"])


def test_exact_small_integers():
    """Rows of small integers and weights 1/4: every partial and every sum is
    exact in bf16 / fp32, so y == x exactly, on any rank split."""
    rng = np.random.default_rng(2)
    T, H, E, R, k = 40, 64, 32, 8, 4
    xf = rng.integers(-8, 9, (T, H)).astype(np.float32)
    x = W.f32_to_bf16_bits(xf)
    idx = np.argsort(rng.random((T, E)), 1)[:, :k].astype(np.int64)
    w = np.full((T, k), 0.25, np.float32)
    sr = oracle.slots_ranks(idx, w, E, R)
    rx = oracle.dispatch_rows(x, sr["token_rank_slot"], rows=T * min(k, R))
    part = oracle.expert_reduce_ranks(idx, w, E, R, sr["rank_offset"], sr["recv_src_idx"], rx)
    y = oracle.combine_ranks(part, sr["token_rank_slot"])
    np.testing.assert_array_equal(y, x)
    # a partial is x times the share of the token's experts on that rank
    epr = E // R
    for t in range(3):
        for r in range(R):
            s = sr["token_rank_slot"][t, r]
            if s >= 0:
                n = int(((idx[t] // epr) == r).sum())
                np.testing.assert_array_equal(oracle.bf16_to_f32(part[s]), xf[t] * (0.25 * n))


def _ulp_bf16(v):
    a = np.abs(v.astype(np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


@pytest.mark.parametrize("fmt,expert", [("bf16", "identity"), ("bf16", "scale"), ("fp8", "identity"),
                                        ("fp8", "scale")])
def test_rounding_bound(fmt, expert):
    """|y - exact| <= half an ulp of y, plus half an ulp of each partial
    (times nothing: partials enter the sum unweighted), plus half an ulp of
    each expert output element times its weight; exact = fp64 sum over the
    token's valid slots of w * v * s_e, with v the received element."""
    inp = W.make_inputs("prefill2n", T=96, H=256, x_fmt=fmt, expert=expert, mask_frac=0.1)
    if expert == "scale":
        inp["expert_factor"] = np.random.default_rng(4).uniform(0.5, 1.5, inp["E"]).astype(np.float32)
    out = oracle.run_path(dict(inp, rank_rows=True))
    idx, w, E, R = inp["topk_idx"], inp["topk_w"], inp["E"], inp["R"]
    if fmt == "fp8":
        v = (oracle.e4m3_to_f32(out["x_q"]).astype(np.float64)
             * np.repeat(out["x_scales"].astype(np.float64), 128, axis=1))
    else:
        v = oracle.bf16_to_f32(inp["x"]).astype(np.float64)
    fac = inp["expert_factor"] if expert == "scale" else np.ones(E, np.float32)
    T, H = v.shape
    exact = np.zeros((T, H))
    slack = np.zeros((T, H))
    for j in range(inp["k"]):
        ok = idx[:, j] >= 0
        e = np.where(ok, idx[:, j], 0)
        o = v * fac[e].astype(np.float64)[:, None]
        exact += np.where(ok[:, None], w[:, j, None].astype(np.float64) * o, 0.0)
        slack += np.where(ok[:, None], w[:, j, None] * 0.5 * _ulp_bf16(o), 0.0)
    y = oracle.bf16_to_f32(out["y"]).astype(np.float64)
    trs = out["slots"]["token_rank_slot"]
    part = oracle.bf16_to_f32(out["expert_out"]).astype(np.float64)
    for r in range(R):
        s = trs[:, r]
        ok = s >= 0
        slack += np.where(ok[:, None], 0.5 * _ulp_bf16(part[np.where(ok, s, 0)]), 0.0)
    bound = 0.5 * _ulp_bf16(y) + slack * (1 + 1e-5) + 1e-30
    err = np.abs(y - exact)
    assert (err <= bound).all(), float((err - bound).max())
    # the bound is not vacuous: most elements sit well inside it
    assert np.median(err / bound) < 0.5


def test_masked_token_gets_positive_zero():
    inp = W.make_inputs("tiny", mask_tokens=0.2)
    out = oracle.run_path(dict(inp, rank_rows=True))
    dead = (inp["topk_idx"] < 0).all(axis=1)
    assert dead.any()
    assert (out["y"][dead] == 0).all()
    assert (out["slots"]["token_rank_slot"][dead] == -1).all()
