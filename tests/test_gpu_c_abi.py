"""The C ABI used from C++ alone: tests/c/abi_driver (built by
__graft_entry__.build()) allocates its buffers with hipMalloc, runs route ->
dispatch -> stand-in expert -> combine and the fused route + dispatch on
three small seeded layers (128-value scales; one scale per token with a
shared expert and replicas; a one-launch decode batch with softmax gates)
and checks the layout invariants, the fused call's equality with the two
calls, and the argument checks.  Started as a child process."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "_build", "abi_driver")


def test_c_abi_driver_route_dispatch_combine():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build() first")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr + r.stdout
    assert "abi driver ok" in r.stdout
