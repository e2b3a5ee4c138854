"""The C ABI used from a plain C program (tests/c/c_caller.c): host-side
checks without a GPU, and a chunked forward plus a decode step on the GPU
against the fp64 oracle."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c"))
import build_c_caller  # noqa: E402


def _binary():
    if not os.path.exists(build_c_caller.BIN):
        build_c_caller.build()
    return build_c_caller.BIN


def test_c_caller_host_checks():
    r = subprocess.run([_binary(), "cpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.gpu
def test_c_caller_forward_backward_and_decode_on_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(build_c_caller.BIN), "build the C caller first (__graft_entry__.build())"
    print("[gpu case] C caller forward + backward + decode", file=sys.stderr, flush=True)
    r = subprocess.run([build_c_caller.BIN, "gpu"], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
