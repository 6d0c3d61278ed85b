"""The C ABI from a plain C99 program (tests/c_abi/closed_form.c, built by
__graft_entry__.build()): decode in fp32 and bf16 over ragged lengths (with
empty and one-key sequences) and causal and full bf16 prefill, all with
all-zero keys so the exact answer is the mean of the visible values; the
partial merge on partials whose exact merge is known; argument errors and
bit-identical repeats. The program runs as a child process and exits 0 when
every check passes."""
import os
import subprocess

import pytest

from _gpu import needs_gpu

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi", "closed_form")


@pytest.mark.gpu
@needs_gpu
def test_c_caller_closed_forms():
    assert os.path.exists(EXE), "build the C caller first: python -c 'import __graft_entry__ as g; g.build()'"
    print("running", EXE, flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def test_c_caller_is_valid_c99():
    # the header and the caller compile as strict C99 with every warning an error
    import importlib.util
    spec = importlib.util.spec_from_file_location("c_abi_build", os.path.join(HERE, "c_abi", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    r = subprocess.run(["gcc"] + b.CFLAGS + ["-fsyntax-only", b.SRC], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
