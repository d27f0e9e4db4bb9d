"""GPU: the plain-C driver (tests/c/abi_round.c) runs one round through the
C ABI without Python and checks each step's structural facts on the host
(ranked top-K rows, a prefix-closed score-ordered tree with ancestor-or-self
mask rows, root attention against a direct fp64 sum, the walk, the
compacted rows). build() compiles it next to its source."""
import os
import subprocess

import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu

DRIVER = os.path.join(os.path.dirname(__file__), "c", "abi_round")


def test_c_driver_round():
    if not os.path.exists(DRIVER):
        raise FileNotFoundError(f"{DRIVER} is missing: run __graft_entry__.build() first")
    say("c driver abi_round")
    res = subprocess.run([DRIVER], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi_round ok" in res.stdout
