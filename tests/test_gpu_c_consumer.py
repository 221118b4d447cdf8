"""The library used from C alone: tests/c_api/abi_consumer (built by the
package build) runs one causal bf16 forward and its backward through
include/flash_attn.h on HIP device buffers, checks both against the fp64
oracle (O within 2e-2, LSE within 1e-2; each gradient within
2e-2 * max(1, max |g_ref|) and an RMS error of 1e-2 of its RMS) and three
synchronous error returns."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_api", "abi_consumer")


def test_c_consumer_runs():
    if not os.path.exists(EXE):
        pytest.fail("tests/c_api/abi_consumer is not built (run __graft_entry__.build())")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK")
