"""Build libmoe_mxfp4.so (the C-ABI library) from csrc/*.hip with hipcc for gfx950.

Run ``python -m mxfp4_weights_fp8_amd.build`` (or ``__graft_entry__.build()``).
The library lands next to this file; object files go to ``_build/``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_mxfp4.so")
SOURCES = ["moe_api.hip", "plan.hip", "quant.hip", "pack.hip", "gemm_small.hip", "gemm_large.hip", "gemm_xl.hip",
           "gemm_fewk.hip", "gemm_dense.hip", "gemm_chain.hip", "gemm_a16.hip", "combine.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: never emit v_pk_{add,mul,fma}_f32 (the host pass warns that it
# does not know the feature; that is harmless).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source extras. The LDS-staged GEMMs keep their 128 accumulator registers in the
# unified VGPR file: with MFMA results in AGPRs, the register allocator rotates
# accumulators through copies inside the K loop (v_accvgpr moves between dependent
# MFMAs), which halves the MFMA issue rate.
EXTRA = {"gemm_large.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "gemm_fewk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "gemm_dense.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build_test_support(verbose: bool = False) -> str:
    """Compile the test-support library tests/native/libmfma_probe.so (single-MFMA
    probes the GPU tests use to check the hardware dot product; not part of the
    product library)."""
    root = os.path.dirname(HERE)
    src = os.path.join(root, "tests", "native", "mfma_probe.hip")
    out = os.path.join(root, "tests", "native", "libmfma_probe.so")
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    build_test_support(verbose=True)
    sys.exit(0)
