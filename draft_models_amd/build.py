"""Build libmla.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Usage: python -m draft_models_amd.build   (or draft_models_amd.build.build())
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmla.so")
BUILD_DIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# packed-fp32 instructions are disabled: the compiler may otherwise form
# v_pk_{add,mul,fma}_f32 from ordinary float code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(PKG, "..", "include")]


# Per-file code-generation options. The stream-K decode keeps its latent
# output accumulators in VGPRs (its rare rescale multiplies them there) and its
# queries in AGPRs; with the VGPR form of MFMA the accumulators are not moved
# between the two register files every tile.
FILE_FLAGS = {"attn_decode_sk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx950 target feature; that warning is expected
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


PEAKS_SRC = os.path.join(PKG, "peaks", "peaks.hip")
PEAKS_OUT = os.path.join(PKG, "libmla_peaks.so")


def build_peaks(verbose: bool = True) -> str:
    """libmla_peaks.so: the measured-roofline kernels (copy, read, MFMA loop)
    used by bench.py; separate from the MLA library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = _compile(PEAKS_SRC)
    tmp = PEAKS_OUT + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", obj, "-o", tmp], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, PEAKS_OUT)
    if verbose:
        print(f"built {PEAKS_OUT}")
    return PEAKS_OUT


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
    build_peaks()
