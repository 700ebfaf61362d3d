"""The C ABI from plain C: tests/c_abi/ep_c_check (built by
__graft_entry__.build() with gcc and the HIP runtime only) runs layout ->
dispatch -> combine and the single-call layout + dispatch through
libep_hip.so and compares every output with the C oracle."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi", "ep_c_check")


def test_c_program_matches_oracle():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(BIN), "tests/c_abi/ep_c_check is not built (run __graft_entry__.build())"
    print("running", BIN, flush=True)
    p = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(p.stdout, p.stderr, flush=True)
    assert p.returncode == 0, p.stdout + p.stderr
    assert p.stdout.count("match") == 2
