"""The forward through the C ABI from a plain C program (tests/c_abi_fwd.c): device
memory from hipMalloc, bsattn_fwd on its own stream, results against the fp64
oracle -- the library used with no Python or torch in the process."""
import subprocess
import sys

import pytest

import c_abi_build
from gpu_util import ensure_built, say

pytestmark = pytest.mark.gpu


def test_c_program_forward():
    ensure_built()
    import oracle
    oracle.build(force=False)
    exe = c_abi_build.build(force=False)
    say("c_abi_fwd", exe)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    sys.stdout.write(r.stdout)
    sys.stderr.write(r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("PASS") == 3
