"""attn_fwd called from a plain C11 program (tests/c_abi/attn_fwd_c.c, built
by the package build next to the library): hipMalloc'd buffers, a HIP
stream, and closed-form checks of the output (one key gives that key's value
row bit for bit; constant value rows give that constant)."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "scaled_dot_product_16_amd", "_build", "attn_fwd_c")


@pytest.mark.skipif(not os.path.exists(EXE), reason="the C caller is built by the package build (needs gcc)")
def test_c_caller_runs_attn_fwd():
    print("[c abi] attn_fwd from C", flush=True)
    sys.stdout.flush()
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
