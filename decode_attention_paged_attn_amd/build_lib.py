"""Compile the HIP library in-tree for gfx950.

``python -m decode_attention_paged_attn_amd.build_lib`` (or ``build()``) runs
hipcc on each HIP source under ``csrc/`` (in parallel, one object each) and
links the objects into ``libpagedattn.so`` next to this file.  It always
recompiles.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpagedattn.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # device code never relies on NaN propagation (tails are masked by select),
    # so max reductions fuse into single DPP instructions
    "-Xarch_device", "-fno-honor-nans",
    "-Wall",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _filter(text):
    return "\n".join(line for line in text.splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in line)


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return res.returncode, _filter(res.stdout)


def build(verbose=False, extra_flags=(), jobs=None):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with tempfile.TemporaryDirectory(prefix="pda_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in srcs]
        cmds = [[hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-c", s, "-o", o]
                for s, o in zip(srcs, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, out), s in zip(results, srcs):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {os.path.basename(s)} ({rc}):\n{out}")
            if verbose and out.strip():
                print(out, flush=True)
        tmp = LIB + ".tmp"
        link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        rc, out = _run(link)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{out}")
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB)
    sys.exit(0)
