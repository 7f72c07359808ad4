"""The C ABI driven from a plain C program (tests/native/c_abi_driver.c): HIP
memory and a HIP stream of its own, host- and device-built plans with both
selections, every exchange form, compared bit for bit with the C oracle. No
Python binding and no torch in the process that calls the library."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "native", "_build", "c_abi_driver")

pytestmark = pytest.mark.gpu


def test_c_program_through_the_abi():
    assert os.path.exists(DRIVER), "build first: python -c 'import __graft_entry__ as g; g.build()'"
    print("[gpu] running the C ABI driver", flush=True)
    sys.stdout.flush()
    r = subprocess.run([DRIVER], capture_output=True, text=True, timeout=120)
    print(r.stdout[-3000:])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "all cases bitwise equal to the oracle" in r.stdout
