"""The C ABI from a plain C program (tests/c_abi/abi_check.c, built by
__graft_entry__.build() into _build/abi_check): HIP runtime memory and
stream, the library's calls as the header declares them, results checked
against the oracle inside the program."""
import os
import subprocess

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "_build", "abi_check")


def test_c_program_drives_the_abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(BIN), "_build/abi_check missing: run __graft_entry__.build()"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "abi_check ok" in r.stdout
