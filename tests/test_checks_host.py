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


PLAN = os.path.join(ROOT, "tests", "host", "plan_driver.cpp")


def _build_plan(tmp_path):
    exe = str(tmp_path / "plan")
    r = subprocess.run(["g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", PLAN, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_decode_chunk_choice_on_host(tmp_path):
    """choose_chunk (the decode planner's chunk) over seeded length
    distributions: chunk in range, items within the partial buffers' capacity,
    never costlier than the k-candidates alone."""
    r = subprocess.run([_build_plan(tmp_path), "sweep"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert int(r.stdout.split()[1]) == 0 and int(r.stdout.split()[3]) > 10_000, r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_decode_chunk_choice_ragged_v3(tmp_path):
    """On the seeded paged ragged workload (B=128, lengths U{512..32768}, 256
    CUs, 256-token minimum chunk, the bf16 partial overhead, a round costing
    H + 512 rows besides its tokens) the plan takes two rounds of at most
    4864 tokens: chunk total/(4 CUs) rounded up would leave 55 work-groups
    with a fifth round (5 x 2144 = 10720 tokens)."""
    import numpy as np
    from mla_latent_kv_22_amd import inputs as I
    lens = I.seq_lengths(I.RAGGED, np.random.default_rng(0))
    ovh = int(2 * 128 * (512 * 2 + 8) / (576 * 2))
    r = subprocess.run([_build_plan(tmp_path), "plan", "256", "256", str(ovh), str(128 + 512)],
                       input=" ".join(map(str, lens)), capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    ch, items, rounds = map(int, r.stdout.split())
    assert ch % 32 == 0 and rounds == 2 and rounds * ch <= 9728, r.stdout
    # the uniform V3 batch keeps its exact one-round plan
    r = subprocess.run([_build_plan(tmp_path), "plan", "256", "256", str(ovh), str(128 + 512)],
                       input=" ".join(["8192"] * 64), capture_output=True, text=True, timeout=60)
    assert r.stdout.split() == ["2048", "256", "1"], r.stdout
