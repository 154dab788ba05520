"""Build liblowram.so (gfx950) in-tree with hipcc.

Every .hip source under csrc/ is compiled to an object in parallel and linked
into one shared library next to this file.  The packed-fp32 feature is
switched off for device code (the host pass warns that it does not know the
feature; that warning is harmless).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblowram.so")
BUILD = os.path.join(HERE, "_build")
PEAKS_SRC = os.path.join(HERE, "peaks")
PEAKS_LIB = os.path.join(HERE, "libpeaks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-Wno-unknown-warning-option"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build_peaks(verbose: bool = False) -> str:
    """libpeaks.so: the benchmark's achievable-peak probes (streaming read,
    MFMA loop), kept out of the decode library."""
    src = os.path.join(PEAKS_SRC, "peaks.hip")
    tmp = PEAKS_LIB + ".tmp"
    r = subprocess.run([HIPCC, *FLAGS, "-shared", "-o", tmp, src], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    os.replace(tmp, PEAKS_LIB)
    if verbose:
        print("built", PEAKS_LIB)
    return PEAKS_LIB


def build(verbose: bool = False) -> str:
    build_peaks(verbose)
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
