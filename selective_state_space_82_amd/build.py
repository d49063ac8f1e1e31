"""Build libssmscan.so in-tree with hipcc for gfx950 (always recompiles)."""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libssmscan.so")
SOURCES = ["scan_fwd.hip", "scan_small.hip", "agg_rev.hip", "scan_bwd.hip", "scan_step.hip", "conv1d.hip", "lti.hip", "ssd.hip",
           "ssd_scan.hip", "noalloc.hip", "abi.cpp"]
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


# The sources that decide the prefill kernels and their launch shapes.
FWD_KERNEL_SOURCES = ("abi.cpp", "agg_rev.hip", "device_common.h", "launch.h", "scan_fwd.hip", "scan_small.hip",
                      "tile_common.h")
# The sources behind each group of kernels a profile under profiles/ covers.
PROFILE_SOURCES = {
    "scan_fwd": FWD_KERNEL_SOURCES,
    "scan_step": ("abi.cpp", "device_common.h", "launch.h", "scan_step.hip"),
    "scan_bwd": ("abi.cpp", "agg_rev.hip", "device_common.h", "launch.h", "scan_bwd.hip", "scan_fwd.hip",
                 "tile_common.h"),
    "conv1d": ("abi.cpp", "device_common.h", "launch.h", "conv1d.hip", "tile_common.h"),
    "frontend": ("abi.cpp", "conv1d.hip", "device_common.h", "launch.h", "scan_fwd.hip", "tile_common.h"),
    "lti": ("abi.cpp", "device_common.h", "launch.h", "lti.hip", "tile_common.h"),
    "ssd": ("abi.cpp", "device_common.h", "launch.h", "ssd.hip", "ssd_common.h", "ssd_scan.hip"),
}


def kernel_source_hash(names=FWD_KERNEL_SOURCES) -> str:
    """sha256 over the named library sources (default: those of the prefill kernels), identifying which
    kernels a stored measurement belongs to."""
    h = hashlib.sha256()
    for name in sorted(names):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile(src: str, out_dir: str) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + COMMON + ["-c"] + lang + [os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
