"""Pins of the oracle's number formats and quantization rules (CPU only).

The formats are fixed by their published definitions:
  - OCP 8-bit floating point, E4M3 (bias 7, 3 mantissa bits, S.1111.111 NaN,
    no infinities, max 448), round to nearest even, saturating;
  - OCP Microscaling E8M0 scale (2^(e-127), 0xFF NaN);
  - bfloat16 round to nearest even.
The pages fix the payload shapes: fp8 with one fp32 scale per 128 elements
(MORI-EP Benchmark, Reference script's fp8 factor) and mxfp8 = 32 e4m3 + one
e8m0 (MoE-EP Benchmark README, MEGA_COMBINE_DTYPE).  The expectations below
come from exact rational arithmetic on those definitions and from torch's
own casts, never from the oracle.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from combine_dispatch_layout_02_amd import workloads as W


def e4m3_value(code: int):
    """Exact value of an e4m3 code from the format definition (None = NaN)."""
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        return None
    mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -mag if s else mag


def test_e4m3_decode_all_codes():
    dec = oracle.e4m3_to_f32(np.arange(256, dtype=np.uint8))
    for c in range(256):
        v = e4m3_value(c)
        if v is None:
            assert np.isnan(dec[c])
        else:
            assert Fraction(float(dec[c])) == v, hex(c)
            assert np.signbit(dec[c]) == bool(c & 0x80)
    assert float(dec[0x7E]) == 448.0 and float(dec[0x01]) == 2.0 ** -9
    # torch's e4m3fn decode agrees on every code
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(np.isnan(t), np.isnan(dec))
    np.testing.assert_array_equal(t[~np.isnan(t)], dec[~np.isnan(dec)])


def test_e4m3_encode_round_trips_every_finite_code():
    codes = [c for c in range(256) if e4m3_value(c) is not None]
    vals = oracle.e4m3_to_f32(np.array(codes, np.uint8))
    np.testing.assert_array_equal(oracle.f32_to_e4m3(vals), np.array(codes, np.uint8))


def test_e4m3_midpoints_round_to_even_and_neighbours_to_nearest():
    pos = sorted({e4m3_value(c) for c in range(128) if e4m3_value(c) is not None})
    code_of = {e4m3_value(c): c for c in range(128) if e4m3_value(c) is not None}
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = (lo + hi) / 2
        assert Fraction(float(np.float32(mid))) == mid  # midpoints are exact in fp32
        even = code_of[lo] if code_of[lo] % 2 == 0 else code_of[hi]
        assert oracle.f32_to_e4m3(np.float32(mid)) == even
        assert oracle.f32_to_e4m3(-np.float32(mid)) == even | 0x80
        below = np.nextafter(np.float32(mid), np.float32(0))
        above = np.nextafter(np.float32(mid), np.float32(1e9))
        assert oracle.f32_to_e4m3(below) == code_of[lo]
        assert oracle.f32_to_e4m3(above) == code_of[hi]


def test_e4m3_saturation_nan_zero():
    for v in (448.0, 449.0, 463.99, 464.0, 464.01, 480.0, 1e6, 3.4e38, np.inf):
        assert oracle.f32_to_e4m3(np.float32(v)) == 0x7E, v
        assert oracle.f32_to_e4m3(np.float32(-v)) == 0xFE, v
    assert oracle.f32_to_e4m3(np.float32(np.nan)) & 0x7F == 0x7F
    assert oracle.f32_to_e4m3(np.float32(0.0)) == 0x00
    assert oracle.f32_to_e4m3(np.float32(-0.0)) == 0x80
    assert oracle.f32_to_e4m3(np.float32(2.0 ** -11)) == 0x00        # below half the min subnormal
    assert oracle.f32_to_e4m3(np.float32(2.0 ** -10)) == 0x00        # tie with 0 -> even (0)
    assert oracle.f32_to_e4m3(np.float32(3 * 2.0 ** -11)) == 0x01    # nearest is 2^-9
    assert oracle.f32_to_e4m3(np.float32(1e-45)) == 0x00             # fp32 subnormal input


def test_e4m3_matches_torch_cast_in_range():
    rng = np.random.default_rng(0)
    mags = np.exp2(rng.uniform(-14, np.log2(463.9), 40000)).astype(np.float32)
    vals = mags * np.where(rng.random(40000) < 0.5, -1, 1).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.f32_to_e4m3(vals), ref)


def test_e8m0_all_codes():
    dec = oracle.e8m0_to_f32(np.arange(256, dtype=np.uint8))
    for e in range(255):
        assert Fraction(float(dec[e])) == Fraction(2) ** (e - 127)
    assert np.isnan(dec[255])
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).float().numpy()
    np.testing.assert_array_equal(t[:255], dec[:255])


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, 30000, dtype=np.uint64).astype(np.uint32)
    # add exact midpoints (low half 0x8000) with even and odd kept parts, and edges
    special = np.array([0x3F808000, 0x3F818000, 0x7F7F8000, 0x7F7FFFFF, 0x00008000,
                        0x00018000, 0x80008000, 0x7F800000, 0xFF800000, 0x00000001], np.uint32)
    bits = np.concatenate([bits, special, bits[:2000] & 0xFFFF8000 | 0x8000])
    f = bits.view(np.float32)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(f)
    nan = np.isnan(f)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert (got[nan] == 0x7FC0).all()
    back = oracle.bf16_to_f32(got[~nan])
    np.testing.assert_array_equal(back.view(np.uint32), got[~nan].astype(np.uint32) << 16)


def test_fp8_factor_and_row_bytes():
    H = 7168
    assert (1 + 4 / 128) / 2 == 0.515625
    assert H + 4 * (H // 128) == 2 * H * 0.515625 == 7392


def test_quant_fp8_s128_rule():
    inp = W.make_inputs("quant", T=16, H=1024)
    x = inp["x"].copy()
    x[3, 128:256] = 0          # an all-zero group
    q, s = oracle.quant_fp8_s128(x)
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    amax = xf.view(16, -1, 128).abs().amax(-1)
    scale_ref = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    np.testing.assert_array_equal(s, scale_ref.numpy())
    assert s[3, 1] == 1.0 and (q[3, 128:256] & 0x7F == 0).all()
    ratio = (xf.view(16, -1, 128) / scale_ref[..., None]).view(16, -1)
    assert ratio.abs().max() < 464  # torch's cast would give NaN from 464 on; our rule saturates
    ref = ratio.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q, ref)
    # every group's largest magnitude lands on +-448
    assert ((q.reshape(16, -1, 128) & 0x7F).max(-1)[amax.numpy() > 0] == 0x7E).all()


def test_quant_mxfp8_rule():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal((8, 512)) * np.exp2(rng.integers(-20, 20, (8, 1)))).astype(np.float32)
    v[0, :32] = 0.0
    v[1, :32] = 1e-40   # fp32 subnormals
    v[2, :32] *= 1e30
    q, e = oracle.quant_mxfp8(v)
    assert e[0, 0] == 0 and (q[0, :32] & 0x7F == 0).all()
    for r in range(8):
        for g in range(512 // 32):
            grp = v[r, g * 32:(g + 1) * 32]
            amax = float(np.abs(grp).max())
            if amax == 0:
                continue
            X = int(e[r, g]) - 127
            # the shared exponent puts amax in [2^8, 2^9) after scaling (before clamping)
            assert Fraction(2) ** 8 <= Fraction(amax) * Fraction(2) ** -X < Fraction(2) ** 9 or X in (-127, 127)
            scaled = (torch.from_numpy(grp.copy()) * torch.tensor(2.0 ** -X, dtype=torch.float32))
            ref = scaled.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            np.testing.assert_array_equal(q[r, g * 32:(g + 1) * 32], ref)


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_inherent_quantization_error_on_normal_rows():
    """The formats' own error floor on N(0,1) rows (hidden 7168): about 2.6 %
    for per-128 e4m3, 2.9 % for mxfp8 and 3.9 % for the fp8 -> mxfp8 chain,
    all above a 2 % relative-L2 bar measured against unquantized fp32."""
    inp = W.make_inputs("quant", T=32)
    x = inp["x"]
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    q, s = oracle.quant_fp8_s128(x)
    deq8 = oracle.e4m3_to_f32(q).astype(np.float64) * np.repeat(s, 128, axis=1)
    mq, me = oracle.quant_mxfp8(xf.astype(np.float32))
    deqmx = oracle.e4m3_to_f32(mq).astype(np.float64) * np.repeat(oracle.e8m0_to_f32(me), 32, axis=1)
    v = (oracle.e4m3_to_f32(q) * np.repeat(s, 128, axis=1)).astype(np.float32)
    cq, ce = oracle.quant_mxfp8(v)
    chain = oracle.e4m3_to_f32(cq).astype(np.float64) * np.repeat(oracle.e8m0_to_f32(ce), 32, axis=1)
    assert abs(_rel_l2(deq8, xf) - 0.026) < 0.003
    assert abs(_rel_l2(deqmx, xf) - 0.029) < 0.003
    assert abs(_rel_l2(chain, xf) - 0.039) < 0.003


# ---------------------------------------------------------------- e2m1 / nvfp4

def e2m1_value(code: int) -> Fraction:
    """OCP E2M1 from its definition: bias 1, one mantissa bit, field 0 subnormal."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return -mag if s else mag


def e2m1_nearest(x: float) -> int:
    """Brute force: the code whose value is nearest to x; ties go to the code
    with an even mantissa bit; beyond the largest magnitude, saturate."""
    fx = Fraction(float(x))
    best = None
    for c in range(16):
        if (c & 8) != (8 if np.signbit(x) else 0):
            continue
        d = abs(e2m1_value(c) - fx)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_e2m1_decode_all_codes():
    dec = oracle.e2m1_to_f32(np.arange(16, dtype=np.uint8))
    assert [Fraction(float(v)) for v in dec] == [e2m1_value(c) for c in range(16)]
    assert sorted({abs(float(v)) for v in dec}) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e2m1_encode_against_brute_force():
    grid = np.concatenate([np.linspace(-7, 7, 2801), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 6.0, 1e30,
                                                      -1e-30, -0.0]]).astype(np.float32)
    np.testing.assert_array_equal(oracle.f32_to_e2m1(grid), [e2m1_nearest(v) for v in grid])


def test_quant_nvfp4_rule():
    import torch
    rng = np.random.default_rng(6)
    v = (rng.standard_normal((4, 256)) * np.exp2(rng.integers(-10, 10, (4, 1)))).astype(np.float32)
    v[0, :16] = 0.0
    q, s = oracle.quant_nvfp4(v)
    for r in range(4):
        for g in range(16):
            grp = v[r, g * 16:(g + 1) * 16]
            amax = torch.tensor(float(np.abs(grp).max()), dtype=torch.float32)
            sb = int((amax / 6.0).to(torch.bfloat16).view(torch.int16)) & 0xFFFF
            if sb & 0x7FFF == 0:
                sb = 0x3F80
            assert s[r, g] == sb
            sf = np.uint32(sb << 16).view(np.float32)
            codes = [(q[r, (g * 16 + i) // 2] >> (4 * (i % 2))) & 0xF for i in range(16)]
            assert codes == [e2m1_nearest(np.float32(x) / sf) for x in grp]


def test_nvfp4_combine_matches_fp64_and_representable_rows():
    inp = W.make_inputs("nvfp4", T=48, H=512, E=32, R=8)
    out = oracle.run_path(inp)
    ts, w = out["slots"]["token_slot"], inp["topk_w"]
    codes = np.stack([(out["expert_q"] >> 0) & 0xF, (out["expert_q"] >> 4) & 0xF], axis=-1).reshape(
        out["expert_q"].shape[0], -1)
    deq = oracle.e2m1_to_f32(codes).astype(np.float64)
    sc = (out["expert_scales"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    deq *= np.repeat(sc, 16, axis=1)
    y64 = np.zeros((ts.shape[0], deq.shape[1]))
    for t in range(ts.shape[0]):
        for j in range(ts.shape[1]):
            y64[t] += float(w[t, j]) * deq[ts[t, j]]
    import torch
    ref = torch.from_numpy(y64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    def ordered(x):
        x = np.asarray(x, np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    assert np.abs(ordered(out["y"]) - ordered(ref)).max() <= 1
    # rows made of e2m1 values with a 6 in every group (scale exactly 1) survive
    rng = np.random.default_rng(8)
    vals = oracle.e2m1_to_f32(rng.integers(0, 16, (16, 256)).astype(np.uint8))
    vals[:, ::16] = 6.0
    x = W.f32_to_bf16_bits(vals)
    idx = np.argsort(rng.random((16, 8)), 1)[:, :4].astype(np.int64)
    wt = np.full((16, 4), 0.25, np.float32)
    res = oracle.run_path(dict(T=16, H=256, E=8, R=4, N=1, k=4, x=x, topk_idx=idx, topk_w=wt,
                               x_fmt="bf16", y_fmt="nvfp4", expert="identity"))
    np.testing.assert_array_equal(res["y"], x)
