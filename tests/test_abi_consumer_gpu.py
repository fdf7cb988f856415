"""The library used from a C++ program through include/pva.h and the HIP
runtime only (tests/host/abi_consumer.cpp, built by __graft_entry__.build()
next to its source): descriptor, device buffers, the bf16 forward, and
closed forms of the masked softmax (with K = 0 every row is the mean of the V
rows it sees; text row 0 is v_0 bitwise), the useful-FLOP count and the
argument errors."""
import os
import subprocess

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host", "abi_consumer")


def test_cpp_program_through_the_c_abi():
    assert os.path.exists(EXE), "tests/host/abi_consumer is missing: run __graft_entry__.build() first"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_consumer: ok" in r.stdout
