"""Build ``libmoe.so`` (gfx950) in-tree with hipcc.

Usage: ``python combine_router_softmax_amd/build.py`` (or ``build()``).
Every ``csrc/*.hip`` file is compiled to an object in parallel, then linked
into ``combine_router_softmax_amd/libmoe.so``. ``probes/ceilings.hip`` (the
measured-ceilings program that ``bench.py --ceilings`` runs) is built beside
it as ``combine_router_softmax_amd/ceilings``, and ``probes/fp8_encode.hip``
(the exhaustive check of the e4m3 encoder that a GPU test runs) as
``combine_router_softmax_amd/fp8_encode_check``.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
PROBE_SRC = os.path.join(PKG, "probes", "ceilings.hip")
PROBE = os.path.join(PKG, "ceilings")
FP8_PROBE_SRC = os.path.join(PKG, "probes", "fp8_encode.hip")
FP8_PROBE = os.path.join(PKG, "fp8_encode_check")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libmoe.so)")


def _compile(src: str, hipcc: str, verbose: bool) -> str:
    obj = os.path.join(OBJ, os.path.basename(src).replace(".hip", ".o"))
    cmd = [hipcc, *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library. Returns its path."""
    hipcc = _hipcc()
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    jobs = max(1, min(len(srcs), 16, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    _build_probe(hipcc, PROBE_SRC, PROBE)
    _build_probe(hipcc, FP8_PROBE_SRC, FP8_PROBE)
    return LIB


def _build_probe(hipcc: str, src: str, exe: str) -> None:
    tmp = exe + ".tmp"
    cmd = [hipcc, *[f for f in HIPCC_FLAGS if f not in ("-fPIC", "-fvisibility=hidden")], f"-I{CSRC}", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}{r.stderr}")
    os.replace(tmp, exe)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
