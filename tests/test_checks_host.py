"""The device-side index checks and length clamps of the kernels
(csrc/mla_checks.h), compiled for the host with g++ and run over valid and
corrupted block tables, slots and prefill offsets: no result may leave the
caller's buffers, and no valid value may change.  This is the CPU proof of
the predicates the MLA_DEBUG build runs on the device."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "host", "checks_driver.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_check_predicates_on_host(tmp_path):
    exe = str(tmp_path / "checks")
    r = subprocess.run(["g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", DRIVER, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    v, n = r.stdout.split()[1], r.stdout.split()[3]
    assert int(v) == 0 and int(n) > 1_000_000, r.stdout
