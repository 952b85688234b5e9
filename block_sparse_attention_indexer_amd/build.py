"""Build libmsa.so in-tree with hipcc for gfx950.

    python -m block_sparse_attention_indexer_amd.build

Each HIP translation unit is compiled in parallel, then linked into
``block_sparse_attention_indexer_amd/lib/libmsa.so``.  The library has no
dependency on torch; it links only the HIP runtime.
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
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmsa.so")
ARCH = "gfx950"

SOURCES = ["msa_indexer.hip", "msa_attention.hip", "msa_prefill.hip", "msa_latent.hip",
           "msa_noalloc.hip", "msa_errors.hip", "msa_api.cpp"]

# Packed-FP32 VALU ops are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mcode-object-version=5"]

# Per-source flags.  The scorers' MFMA results are read by VALU code (the
# block max) right away; by default the compiler writes them to AGPRs and
# copies them out (96-192 copies per loop in the decode scorer).  Their
# register budget fits everything in VGPRs, so those units select the
# VGPR-result MFMA form (prefill indexer 865 -> 819 us; decode scorers
# unchanged, being HBM-bound).  The latent kernel needs its AGPRs.
#
# msa_prefill.hip also runs its kernels with the IEEE mode bit off
# (-mno-amdgpu-ieee, which requires -fno-honor-nans): in IEEE mode every max
# of an MFMA result first re-quiets it (an extra v_max x, x per element of
# the block-max epilogue and of the softmax).  No NaN reaches a float
# operation there: poisoned or stale slots only ever enter through MFMA
# results that integer-conditioned selects replace by -inf (positions past a
# token, rows past a tile) or V rows zeroed in LDS, before any max, exp or
# sum.  Measured interleaved on the prefill workload: indexer call 0.81 ->
# 0.77 ms, attention call 12.23 -> 11.92 ms, identical block ids.
SOURCE_FLAGS = {
    "msa_indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "msa_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-mno-amdgpu-ieee", "-fno-honor-nans"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str, extra) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
           "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}", *DEVICE_FLAGS, *extra,
           *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")


def build(extra_flags=(), jobs: int = 4) -> str:
    """Compile every source and link libmsa.so; returns the library path."""
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = []
        for s in SOURCES:
            src = os.path.join(CSRC, s)
            obj = os.path.join(objdir, os.path.splitext(s)[0] + ".o")
            objs.append(obj)
            futs.append(ex.submit(_compile, src, obj, SOURCE_FLAGS.get(s, []) + list(extra_flags)))
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC",
           *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
