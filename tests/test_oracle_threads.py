"""The oracle's threaded timing mode produces the bytes of the single-threaded
oracle (CPU).  The benchmark times the oracle on all host cores this way; a
block split that moved a row or dropped a token would show here."""
import numpy as np
import pytest

import oracle
from combine_dispatch_layout_02_amd import workloads as W

CASES = [
    ("tiny", {}),
    ("decode", {"T": 37}),                        # per-expert scaled experts, ragged T
    ("prefill2n", {"T": 301, "H": 512}),
    ("quant", {"T": 129, "H": 256}),               # fp8 rows -> mxfp8 payload
    ("nvfp4", {"T": 77, "H": 256}),
    ("tiny", {"T": 50, "mask_frac": 0.3, "mask_tokens": 0.1, "routing": "replace"}),
    ("tiny", {"T": 3}),                           # fewer tokens than threads
    ("tiny", {"T": 0}),
]


def _same(a, b, path="out"):
    if isinstance(a, dict):
        assert a.keys() == b.keys(), path
        for key in a:
            _same(a[key], b[key], f"{path}.{key}")
    elif isinstance(a, np.ndarray):
        assert a.dtype == b.dtype and a.shape == b.shape, path
        assert a.tobytes() == b.tobytes(), path
    else:
        assert a == b, path


# (token, rank) rows return bf16 partials, so the nvfp4 payload runs token-major only
@pytest.mark.parametrize("name,kw,rank_rows", [(n, kw, rr) for n, kw in CASES for rr in (False, True)
                                               if not (rr and n == "nvfp4")])
def test_threaded_oracle_bytes_equal_single_thread(name, kw, rank_rows):
    inp = dict(W.make_inputs(name, **kw), rank_rows=rank_rows)
    one = oracle.run_path(inp)
    with oracle.threads(7):
        many = oracle.run_path(inp)
    _same(one, many)


def test_threads_context_restores_single_thread():
    with oracle.threads(5):
        assert oracle._THREADS == 5
    assert oracle._THREADS == 1
