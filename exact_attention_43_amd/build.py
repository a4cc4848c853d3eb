"""Build libexattn.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-fp32 instruction selection switched
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass of
hipcc warns that it does not know that feature, which is harmless.  MFMA
accumulators are kept in architectural VGPRs (``-amdgpu-mfma-vgpr-form``), so
the softmax, the O rescale and the backward's P and dS touch them without AGPR
copies; AGPRs then only hold MFMA source operands the allocator moves there.

    python -m exact_attention_43_amd.build          # build
    python -m exact_attention_43_amd.build --check  # also build the host-only checker
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libexattn.so")
ARCH = "gfx950"

HIP_SOURCES = ["fwd_prefill.hip", "fwd_prefill_slots.hip", "fwd_prefill_dsplit.hip", "fwd_decode.hip", "fwd_fp8.hip", "bwd.hip", "exattn_api.cpp"]
HOST_SOURCES = ["validate.cpp"]


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found (ROCm is required to build libexattn)")
    return h


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libexattn.so next to this file; return its path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    common = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
              "-Wno-unused-function"]
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        jobs.append([hipcc, f"--offload-arch={ARCH}", *common, "-Xclang", "-target-feature",
                     "-Xclang", "-packed-fp32-ops",
                     "-mllvm", "-amdgpu-mfma-vgpr-form", *lang, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        jobs.append(["g++", *common, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in HIP_SOURCES + HOST_SOURCES]
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def build_host_checker() -> str:
    """Build the host-only validation code with g++ and ASan/UBSan into a test driver.

    The driver (csrc/validate_check.cpp) exercises every argument check without a GPU.
    """
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "validate_check")
    _run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          f"-I{INCLUDE}", f"-I{CSRC}", os.path.join(CSRC, "validate.cpp"),
          os.path.join(CSRC, "validate_check.cpp"), "-o", exe])
    return exe


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
    if "--check" in sys.argv:
        print(build_host_checker())
