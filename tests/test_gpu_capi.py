"""The C ABI used from plain C (tests/capi_check.c, built by the package's
build script as _build/capi_check): no Python binding and no PyTorch in the
process.  The program checks its own results and prints "capi ok"."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "_build", "capi_check")


def test_c_program_calls_the_library():
    assert os.path.exists(BIN), "capi_check not built: run displaced_patch_parallelism_net_amd/build.py"
    print("[case] plain-C ABI check", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "capi ok" in r.stdout
