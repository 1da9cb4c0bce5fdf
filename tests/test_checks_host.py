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


BLOCKMAP = os.path.join(ROOT, "tests", "host", "blockmap_driver.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_write_absorb_block_map_on_host(tmp_path):
    """The fused write + absorption launch deals its work-groups to roles by
    XCD (mla_checks.h wa_role / wa_grid): every write tile, absorption rank
    and head exactly once, at most two heads per work-group, for every grid
    the host can form."""
    exe = str(tmp_path / "blockmap")
    r = subprocess.run(["g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", BLOCKMAP, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert int(r.stdout.split()[1]) == 0 and int(r.stdout.split()[3]) > 100_000, r.stdout
