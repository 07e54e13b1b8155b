"""Build the HIP libraries for gfx950, in-tree.

    python sparse_attention_long_msa_amd/build.py

compiles ``csrc/*.hip`` into ``libmsa.so`` (the C-ABI library declared in
``include/msa.h``) and ``synth/synth_device.hip`` into ``synth/libmsa_synth.so``
(the device copy of the seeded input generator).  Every call recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmsa.so")
SYNTH_SRC = os.path.join(ROOT, "synth", "synth_device.hip")
SYNTH_LIB = os.path.join(ROOT, "synth", "libmsa_synth.so")

ARCH = os.environ.get("MSA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def _compile(src, obj):
    return _run([HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj])


def build(verbose: bool = False) -> list[str]:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = [(s, os.path.join(BUILD, os.path.basename(s)[:-4] + ".o")) for s in srcs]
    jobs.append((SYNTH_SRC, os.path.join(BUILD, "synth_device.o")))
    workers = min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        logs = list(ex.map(lambda j: _compile(*j), jobs))
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    objs = [o for s, o in jobs if s != SYNTH_SRC]
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    tmp = SYNTH_LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", jobs[-1][1], "-o", tmp])
    os.replace(tmp, SYNTH_LIB)
    return [LIB, SYNTH_LIB]


if __name__ == "__main__":
    for p in build(verbose="-v" in sys.argv):
        print(p)
