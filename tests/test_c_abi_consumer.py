"""The C ABI from a plain C++ program (tests/c_abi/kda_c_consumer.cpp): no
Python binding and no torch between the caller and include/kda.h.  Without a
GPU only the calls that return before any HIP call run; on a GPU the prefill
(fp32 and bf16, with and without an initial state) and a decode step are
checked against the oracle by the program itself."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c_abi", "kda_c_consumer")


def _run(*args, timeout):
    if not os.path.exists(BIN):
        pytest.fail("tests/c_abi/kda_c_consumer is not built (run __graft_entry__.build())")
    r = subprocess.run([BIN, *args], capture_output=True, text=True, timeout=timeout)
    print(r.stdout, end="", flush=True)
    return r


def test_consumer_abi_calls_without_a_gpu():
    r = _run("--abi-only", timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("PASS") == 3 and "FAIL" not in r.stdout


@pytest.mark.gpu
def test_consumer_against_the_oracle():
    r = _run(timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("PASS") == 8 and "FAIL" not in r.stdout
