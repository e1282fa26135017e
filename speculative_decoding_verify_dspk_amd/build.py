"""Build libdspk.so (gfx950) in-tree with hipcc.

    python -m speculative_decoding_verify_dspk_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdspk.so")
PROBE_LIB = os.path.join(PKG, "libdspk_probe.so")      # measurement only: the streaming-read probe
SOURCES = ["qgemm.hip", "slab.hip", "prefill.hip", "pack.hip", "accept.hip", "noalloc.hip", "api.cpp", "plan.cpp", "policy.cpp"]

# Packed fp32 instructions are kept out of every HIP object (the compiler
# would otherwise form them from ordinary float code).
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libdspk.so)")


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + HIP_FLAGS + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stdout}\n{r.stderr}")


def build(out: str = LIB, quiet: bool = True) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda a: _compile(*a), [(os.path.join(CSRC, s), o) for s, o in zip(SOURCES, objs)]))
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    # the benchmark's streaming probe, a library of its own
    pobj = os.path.join(objdir, "probe.hip.o")
    _compile(os.path.join(CSRC, "probe.hip"), pobj)
    ptmp = PROBE_LIB + ".tmp"
    r = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", ptmp, pobj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of the probe failed:\n{r.stdout}\n{r.stderr}")
    os.replace(ptmp, PROBE_LIB)
    if not quiet:
        print(f"built {out} and {PROBE_LIB}")
    return out


if __name__ == "__main__":
    build(quiet=False)
    sys.exit(0)
