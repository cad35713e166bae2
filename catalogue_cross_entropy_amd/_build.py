"""Build librece.so in-tree with hipcc for gfx950 (no torch extension machinery)."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(os.path.dirname(PKG), "_build")
LIB = os.path.join(PKG, "librece.so")
PEAKS_SRC = os.path.join(CSRC, "probes", "peaks.hip")
PEAKS_LIB = os.path.join(PKG, "libpeaks.so")
ARCH = "gfx950"

# Packed float32 instructions are kept out of every kernel (the compiler would
# otherwise form them from ordinary float code).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build_library(jobs: int = 8) -> str:
    """Compile every HIP/C++ source of the package and link librece.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources()))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    _check_stubs(tmp)
    os.replace(tmp, LIB)
    build_peaks()
    return LIB


def _check_stubs(path: str) -> None:
    """Fail when a kernel's host launch stub is missing from the library: hipcc drops
    the stub of a kernel template whose body the host pass cannot instantiate (for
    example a device builtin called straight from a lambda) without an error, and
    the library then fails to load."""
    res = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in res.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        raise RuntimeError("kernel launch stubs missing from the library (host pass failed to instantiate):\n  "
                           + "\n  ".join(missing[:10]))


def build_peaks() -> str:
    """The device peak probes (matrix-core loop, plain copy) as libpeaks.so."""
    os.makedirs(BUILD, exist_ok=True)
    tmp = PEAKS_LIB + ".tmp"
    cmd = [_hipcc(), *HIP_FLAGS, "-shared", PEAKS_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PEAKS_SRC}:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, PEAKS_LIB)
    return PEAKS_LIB


if __name__ == "__main__":
    print(build_library())
