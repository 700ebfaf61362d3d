"""Pins of the oracle's combine (top-k weighted gather-reduce), CPU only.

What fixes the expected values:
  - identity round trip: with identity experts and softmax weights the
    weighted sum is x * sum(w) with sum(w) within a few fp32 ulps of 1, far
    inside half a bf16 ulp, so y must equal x bit for bit (the pages'
    functional tests report a combine difference of 0, MSCCL++ PR 860);
  - fp64 evaluation of the same sum: within one bf16 ulp;
  - a hand-derived case where fp32 accumulation in slot order gives a
    different bf16 result than any other order;
  - masked slots and all-masked tokens.
"""
import numpy as np
import pytest

import oracle
from combine_dispatch_layout_02_amd import workloads as W


def _bf16_to_f64(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)


def _ulp_distance(a_bits, b_bits):
    """Distance in bf16 ulps between two bf16 bit arrays (+0 and -0 equal)."""
    def ordered(x):
        x = np.asarray(x, np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)  # sign-magnitude -> ordered integers
    return np.abs(ordered(a_bits) - ordered(b_bits))


def _bf16_rne_of_f64(v):
    import torch
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("name", ["tiny", "prefill2n"])
def test_identity_round_trip_is_exact(name):
    inp = W.make_inputs(name, T=min(W.WORKLOADS[name]["T"], 512))
    out = oracle.run_path(inp)
    np.testing.assert_array_equal(out["y"], inp["x"])


def test_masked_slots_and_empty_tokens():
    inp = W.make_inputs("tiny", k=4, mask_frac=0.3, mask_tokens=0.1)
    out = oracle.run_path(inp)
    valid = inp["topk_idx"] >= 0
    wsum = np.where(valid, inp["topk_w"], 0).astype(np.float64).sum(axis=1)
    ref = _bf16_to_f64(inp["x"]) * wsum[:, None]
    d = _ulp_distance(out["y"], _bf16_rne_of_f64(ref))
    assert d.max() <= 1
    empty = ~valid.any(axis=1)
    assert empty.any()
    assert (out["y"][empty] == 0).all()  # +0.0 for a token with no valid slot


def test_scaled_experts_within_one_ulp_of_fp64():
    inp = W.make_inputs("decode", T=64)
    out = oracle.run_path(inp)
    y64 = oracle.combine_bf16_f64(out["expert_out"], out["slots"]["token_slot"], inp["topk_w"])
    d = _ulp_distance(out["y"], _bf16_rne_of_f64(y64))
    assert d.max() <= 1
    # the expert stage itself: one fp32 multiply, one RNE (torch's casts as the reference)
    import torch
    rx = torch.from_numpy(out["recv_x"].view(np.int16)).view(torch.bfloat16).float()
    off = out["slots"]["expert_offset"]
    f = np.repeat(inp["expert_factor"], np.diff(off))
    ref = (rx[: off[-1]] * torch.from_numpy(f)[:, None]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(out["expert_out"][: off[-1]], ref)


def test_fp32_slot_order_is_what_is_computed():
    """x = 1.0; w = [1 + 2^-8, 2^-24 x 7].  In slot order the first product
    is the exact bf16 midpoint 1 + 2^-8 and each later 2^-24 is a tie that
    rounds back to it (even), so y = 1.0.  Reversed order accumulates
    7 * 2^-24 first and y = 1 + 2^-7; so does the exact sum."""
    T, H, k = 1, 64, 8
    x = np.full((T, H), 0x3F80, np.uint16)
    w = np.array([[1 + 2.0 ** -8] + [2.0 ** -24] * 7], np.float32)
    slot = np.arange(k, dtype=np.int32).reshape(1, k)
    rows = np.repeat(x, k, axis=0)
    y = oracle.combine_bf16(rows, slot, w)
    assert (y == 0x3F80).all()
    y_rev = oracle.combine_bf16(rows, slot[:, ::-1].copy(), w[:, ::-1].copy())
    assert (y_rev == 0x3F81).all()
    assert (_bf16_rne_of_f64(oracle.combine_bf16_f64(rows, slot, w)) == 0x3F81).all()


def test_mxfp8_combine_matches_fp64_of_dequantized_rows():
    inp = W.make_inputs("quant", T=64, H=1024, E=32, R=8)
    out = oracle.run_path(inp)
    ts, w = out["slots"]["token_slot"], inp["topk_w"]
    deq = oracle.e4m3_to_f32(out["expert_q"]).astype(np.float64)
    sc = oracle.e8m0_to_f32(out["expert_e8m0"]).astype(np.float64)
    deq = deq * np.repeat(sc, 32, axis=1)
    T, k = ts.shape
    y64 = np.zeros((T, deq.shape[1]))
    for t in range(T):
        for j in range(k):
            y64[t] += float(w[t, j]) * deq[ts[t, j]]
    assert _ulp_distance(out["y"], _bf16_rne_of_f64(y64)).max() <= 1


def test_mxfp8_identity_on_exactly_representable_rows():
    """Rows whose values are e4m3 numbers with a significand of at most 1.75
    survive the fp8 -> fp32 -> mxfp8 chain unchanged (the shared exponent
    maps each 32-group's largest magnitude to at most 1.75 * 2^8 = 448), so
    the weighted sum returns x."""
    rng = np.random.default_rng(5)
    T, H, E, k = 16, 256, 8, 4
    codes = rng.integers(0, 0x7E, size=(T, H), dtype=np.uint8)
    codes[(codes & 7) == 7] -= 1  # significand 1.875 would clip under the shared exponent
    codes[:, ::128] = 0x7E  # every 128-group holds 448, so the per-128 scale is 1
    vals = oracle.e4m3_to_f32(codes) * np.where(rng.random((T, H)) < 0.5, -1, 1).astype(np.float32)
    x = W.f32_to_bf16_bits(vals)
    idx = np.argsort(rng.random((T, E)), 1)[:, :k].astype(np.int64)
    logits = rng.standard_normal((T, k)).astype(np.float32)
    wt = np.exp(logits) / np.exp(logits).sum(1, keepdims=True)
    inp = dict(T=T, H=H, E=E, R=4, N=1, k=k, x=x, topk_idx=idx, topk_w=wt.astype(np.float32),
               x_fmt="fp8", expert="identity")
    out = oracle.run_path(inp)
    np.testing.assert_array_equal(out["y"], x)


def test_mxfp8_shared_exponent_clips_significand_1875():
    """Under the OCP shared-exponent rule a group whose largest magnitude has
    significand 1.875 (240 = 1.875 * 2^7) gets X = 7 - 8 = -1, and 240 * 2 =
    480 saturates to 448: the element comes back as 224."""
    v = np.zeros((1, 32), np.float32)
    v[0, 0], v[0, 1] = 240.0, 1.0
    q, e = oracle.quant_mxfp8(v)
    assert int(e[0, 0]) - 127 == -1
    assert q[0, 0] == 0x7E
    assert float(oracle.e4m3_to_f32(q[0, 0])) * 2.0 ** -1 == 224.0
