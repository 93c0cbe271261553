"""Builds libmuon_step.so (HIP kernels for gfx950 + the C-ABI host runtime).

Usage: python -m muon_step_amd.build   (or muon_step_amd.build.build()).
Objects go to _build/ at the repository root; the library is written next to
this file so the in-tree package loads it.
"""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmuon_step.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["runtime.cpp", "elementwise.hip", "ns_gemm_bf16.hip", "ns_gemm_f32.hip", "noalloc.hip"]

# -ffp-contract=off: every fp32 multiply and add of the bookkeeping rounds once.
# packed-fp32-ops disabled: no v_pk_{add,mul,fma}_f32 in device code.
# -fhip-fp32-correctly-rounded-divide-sqrt: fp32 '/' is the IEEE division sequence.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
          f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{INCLUDE}", "-Wall", "-Wno-unused-function"]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose=False):
    """Compiles every source and links the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
