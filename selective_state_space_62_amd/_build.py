"""Build libssscan.so (HIP, gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = PKG / "_build"
LIB = PKG / "libssscan.so"
# the VALU issue-rate probe behind the roofline's constants (bench.py --rates);
# a library of its own, outside the scan's ABI
PROBE_SOURCES = ["valu_rates_probe.hip"]
PROBE_LIB = PKG / "libssprobe.so"

SOURCES = ["api.cpp", "scan_fwd.hip", "scan_bf16_euler.hip", "scan_bf16_zoh.hip", "scan_f32_euler.hip",
           "scan_f32_zoh.hip", "scan_bwd.hip", "scan_bwd_zoh.hip", "state_update.hip", "scan_fwd_noalloc.hip"]
ARCH = "gfx950"

# Packed-FP32 VALU ops are disabled for all device code; see the design notes.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument",
          "-I", str(INCLUDE), "-I", str(CSRC)]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def rocm_include() -> Path:
    return Path(hipcc()).resolve().parent.parent / "include"


def _compile(src: str) -> Path:
    obj = BUILD / (src + ".o")
    path = CSRC / src
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip", "--offload-arch=" + ARCH, *DEVICE_FLAGS, *COMMON, "-c", str(path), "-o", str(obj)]
    else:
        cmd = [hipcc(), "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", str(rocm_include()), *COMMON,
               "-c", str(path), "-o", str(obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def _link(objs, lib: Path) -> None:
    tmp = lib.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> Path:
    """Compile every source for gfx950 and link libssscan.so and the rate probe
    libssprobe.so (always rebuilds)."""
    BUILD.mkdir(exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built", LIB, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
