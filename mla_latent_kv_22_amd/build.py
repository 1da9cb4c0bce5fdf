"""Build libmla.so and libmla_debug.so from csrc/*.hip with hipcc for gfx950
(in-tree).  The debug library is the same sources built with MLA_DEBUG: its
kernels check every block-table entry, slot and device length before use and
report through the device error word (mla_get_device_error).

Usage: python -m mla_latent_kv_22_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmla.so")
LIB_DEBUG = os.path.join(HERE, "libmla_debug.so")
# measurement helper of bench.py (streaming-read ceiling), not part of the ABI
LIB_PROBE = os.path.join(HERE, "libmla_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# per-file extra flags (none at present)
EXTRA = {}


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    obj = os.path.join(OBJ, os.path.basename(src).replace(".hip", "_debug.o" if debug else ".o"))
    cmd = [HIPCC, *FLAGS, *(["-DMLA_DEBUG"] if debug else []), *EXTRA.get(os.path.basename(src), []), "-c", src,
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probe = sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip")))
    jobs = [(s, d) for d in (False, True) for s in srcs] + [(s, False) for s in probe]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    n = len(srcs)
    _link(objs[:n], LIB)
    _link(objs[n:2 * n], LIB_DEBUG)
    _link(objs[2 * n:], LIB_PROBE)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
