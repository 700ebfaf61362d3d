"""The seeded input generators: determinism, shapes, distributions (CPU)."""
import numpy as np
import pytest
import torch

from combine_dispatch_layout_02_amd import workloads as W


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_shapes_and_determinism(name):
    T = min(W.WORKLOADS[name]["T"], 512)
    a = W.make_inputs(name, T=T)
    b = W.make_inputs(name, T=T)
    assert a["x"].dtype == np.uint16 and a["x"].shape == (T, a["H"])
    assert a["topk_idx"].dtype == np.int64 and a["topk_idx"].shape == (T, a["k"])
    assert a["topk_w"].dtype == np.float32 and a["topk_w"].shape == (T, a["k"])
    for key in ("x", "topk_idx", "topk_w"):
        np.testing.assert_array_equal(a[key], b[key])
    c = W.make_inputs(name, T=T, seed=1)
    assert not np.array_equal(a["x"], c["x"])
    # distinct experts per token, all in range
    idx = a["topk_idx"]
    assert ((idx >= 0) & (idx < a["E"])).all()
    assert all(len(set(r)) == a["k"] for r in idx.tolist())
    # softmax weights: positive, sum to 1 within fp32 rounding
    assert (a["topk_w"] > 0).all()
    assert np.abs(a["topk_w"].astype(np.float64).sum(1) - 1).max() < 1e-6


def test_bf16_rows_are_torch_rne_of_normal_draws():
    a = W.make_inputs("tiny")
    rng = np.random.default_rng(0)
    f = rng.standard_normal((a["T"], a["H"]), dtype=np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(a["x"], ref)
    xf = torch.from_numpy(a["x"].view(np.int16)).view(torch.bfloat16).float()
    assert abs(float(xf.mean())) < 0.05 and abs(float(xf.std()) - 1) < 0.05


def test_uniform_routing_is_uniform():
    a = W.make_inputs("prefill2n")
    counts = np.bincount(a["topk_idx"].ravel(), minlength=a["E"])
    mean = a["T"] * a["k"] / a["E"]
    assert np.abs(counts - mean).max() < 6 * np.sqrt(mean)


def test_zipf_routing_is_skewed():
    a = W.make_inputs("skewed", T=2048)
    counts = np.sort(np.bincount(a["topk_idx"].ravel(), minlength=a["E"]))[::-1]
    # the most popular expert is picked by most tokens; the tail is thin
    assert counts[0] > 0.85 * a["T"]
    assert counts[0] > 20 * np.median(counts)


def test_masking_knobs():
    a = W.make_inputs("tiny", k=4, mask_frac=0.3, mask_tokens=0.2)
    idx = a["topk_idx"]
    frac = (idx < 0).mean()
    assert 0.3 < frac < 0.65
    assert (idx < 0).all(axis=1).any()
    r = W.make_inputs("tiny", routing="replace", k=8)
    assert any(len(set(row)) < 8 for row in r["topk_idx"].tolist())
