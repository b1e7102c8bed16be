"""Build the HIP library libzp.so in-tree with hipcc for gfx950.

Every source under csrc/ is compiled to an object with hipcc (device code for
gfx950 only, packed-FP32 instructions disabled) and linked into
``compressed_paged_kv_amd/libzp.so``.  Objects go to ``_build/`` next to
this file.  The benchmark's bandwidth-ceiling kernels (ceilings/) become
``libzp_ceilings.so`` beside it.  ``build()`` always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libzp.so")
# bandwidth ceilings of the box, for the benchmark only (not part of libzp.so)
CEILINGS_SRC = os.path.join(HERE, "ceilings", "ceilings.hip")
CEILINGS_LIB = os.path.join(HERE, "libzp_ceilings.so")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
          "-I", INCLUDE, "-I", CSRC]
# device code must not use packed FP32 instructions (see the design notes)
DEVICE_ONLY = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON]
    if src.endswith(".hip"):
        cmd += DEVICE_ONLY
    cmd += ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs and verbose:
        print(msgs, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    tmp = CEILINGS_LIB + ".tmp"
    cmd = [_hipcc(), *COMMON, *DEVICE_ONLY, "-shared", "-o", tmp, CEILINGS_SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {CEILINGS_SRC}:\n{res.stdout}{res.stderr}")
    os.replace(tmp, CEILINGS_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
