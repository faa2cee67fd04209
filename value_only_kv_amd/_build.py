"""Builds libgva.so (the GVA C-ABI library) in-tree for gfx950.

The host validation/planning code is plain C++ (built by g++, no HIP), the entry points and
kernels are HIP (built by hipcc for gfx950 only), and hipcc links the shared library into
value_only_kv_amd/libgva.so. Objects go to value_only_kv_amd/_build/.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgva.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HIP_SOURCES = ["gva_api.hip", "k_append_absorb.hip", "k_decode_generic.hip", "k_decode_mfma.hip",
               "k_prefill.hip", "k_recon.hip", "k_latent.hip", "k_diag.hip"]
HOST_SOURCES = ["gva_host.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # Packed FP32 instructions stay off: only scalar and float2 source, never v_pk_*_f32.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]
# Per-source additions. The comparator kernel keeps its matrix-core accumulators in ordinary
# vector registers: its vector-ALU code reads every product, and the compiler's default (the
# accumulation registers) adds a copy per value.
HIP_FILE_FLAGS = {"k_recon.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                  "k_latent.hip": ["-Rpass-analysis=kernel-resource-usage"]}
# Sources whose kernels must not use scratch memory: the latent comparator's staging ring waits
# for a fixed count of vector-memory operations, which holds only while its loop issues no
# vector-memory stores (register spills would be such stores). The build reads the compiler's
# resource report and fails when a kernel of these sources has a scratch size.
NO_SCRATCH = {"k_latent.hip"}
GXX_FLAGS = ["-std=c++17", "-O2", "-fPIC", "-Wall", "-Wextra", "-ffp-contract=off",
             "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
             "-I" + os.path.join(ROOT, "include")]


def _hipcc() -> str:
    p = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the GVA library needs ROCm to build")
    return p


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def scratch_users(report: str) -> list:
    """Kernels with a nonzero scratch size in a -Rpass-analysis=kernel-resource-usage report."""
    bad, name = [], None
    for line in report.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:")[1].split()[0]
        elif "ScratchSize [bytes/lane]:" in line:
            if int(line.split("ScratchSize [bytes/lane]:")[1].split()[0]) != 0:
                bad.append(name)
    return bad


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compiles every source and links libgva.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    cmds = []
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmds.append(["g++", *GXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmds.append([hipcc, *HIPCC_FLAGS, *HIP_FILE_FLAGS.get(src, []), "-c",
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 2) // 2), 8)
    srcs = HOST_SOURCES + HIP_SOURCES
    with cf.ThreadPoolExecutor(jobs) as ex:
        for src, out in zip(srcs, ex.map(_run, cmds)):
            if src in NO_SCRATCH:
                bad = scratch_users(out)
                if bad:
                    raise RuntimeError(f"{src}: kernels use scratch memory: {bad}")
                out = ""
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
