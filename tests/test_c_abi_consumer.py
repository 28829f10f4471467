"""The C ABI used from a plain C++ program (tests/c_abi/abi_consumer.cpp,
built by __graft_entry__.build()): hipMalloc'd buffers and a stream of its
own, no Python binding and no torch.  It checks closed forms of the
transform over one-, two- and three-pass default plans in fp32 and fp64,
and the one-pass entry point (fwt_execute_ws) against fwt_execute."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "abi_consumer")


@pytest.mark.gpu
def test_c_abi_consumer():
    assert os.path.exists(EXE), "build the consumer first: __graft_entry__.build()"
    print("[case] C ABI consumer", flush=True)
    sys.stdout.flush()
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=300)
    print(r.stdout[-3000:])
    assert r.returncode == 0 and "abi consumer: ok" in r.stdout, (r.returncode, r.stdout[-3000:],
                                                                  r.stderr[-3000:])


def test_c_abi_consumer_is_built():
    # build() compiles it on the CPU; the GPU run only executes it
    assert os.path.exists(EXE) and os.access(EXE, os.X_OK)
