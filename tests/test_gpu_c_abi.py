"""The C ABI from a plain C program (tests/c_abi/usp_abi_check.c, built by
__graft_entry__.build()): libusp with the HIP runtime and no PyTorch in the
process. The program checks range splits, the relayout round trip bit for
bit (single tensors and several in one launch), the agreement of the
attention entry points bit for bit and error
codes; its exit status is the verdict."""
import os
import subprocess

import pytest

from gpu_util import log

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "usp_abi_check")


@pytest.mark.gpu
def test_plain_c_consumer():
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build() first"
    log("plain C consumer of libusp")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "usp C ABI check: ok" in r.stdout
