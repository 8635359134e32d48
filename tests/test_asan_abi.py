"""The library's host code under AddressSanitizer: tests/asan/abi_driver.cpp calls the C
ABI (argument checks, knobs, status strings; on a GPU also scans, compactions, radix
passes and CSR offsets at sizes that grow the per-stream workspaces, on two streams,
with releases between) from one executable whose host code, the library's included,
is built with -fsanitize=address (device code as in the library)."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DRIVER = os.path.join(HERE, "asan", "abi_driver.cpp")
EXE = os.path.join(HERE, "asan", "abi_asan")
# the executable need not be the first library loaded into the process; leak checking
# is off because the HIP runtime keeps allocations until exit
ENV = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=0:halt_on_error=1")


@pytest.fixture(scope="module")
def exe():
    if not os.path.exists(EXE):
        import sys
        sys.path.insert(0, ROOT)
        from device_wide_prefix_tile_amd import build
        build.build_asan(DRIVER, EXE)
    return EXE


def run(exe, mode, timeout):
    r = subprocess.run([exe, mode], capture_output=True, text=True, timeout=timeout, env=ENV)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and "0 failed checks" in r.stdout, out[-4000:]


def test_host_code_under_asan(exe):
    run(exe, "host", 120)


@pytest.mark.gpu
def test_device_calls_under_asan(exe):
    run(exe, "device", 300)
