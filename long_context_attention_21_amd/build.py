"""Build the HIP library libcsa_mi355x.so for gfx950 (in-tree).

Each source is compiled by hipcc to an object with its own flags, then the
objects are linked into one shared library exporting the C ABI of
include/csa.h.  Run ``python -m long_context_attention_21_amd.build``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INC = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcsa_mi355x.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-result", "-I", INC, "-I", CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = {
    "compress.hip": DEVICE + ["-ffp-contract=off"],
    # no NaN ever reaches these kernels: non-IEEE mode drops the NaN
    # canonicalisation that IEEE-mode max/min would otherwise add
    # MFMA results in VGPRs: the scores feed the exponentials directly and the
    # accumulators need no copies out of AGPRs
    "attend.hip": DEVICE + ["-fno-honor-nans", "-mno-amdgpu-ieee", "-mllvm", "-amdgpu-mfma-vgpr-form"],
    # the score MFMA result feeds VALU code directly: keep it in VGPRs
    "index_topk.hip": DEVICE + ["-ffp-contract=off", "-fno-honor-nans", "-mno-amdgpu-ieee",
                                "-mllvm", "-amdgpu-mfma-vgpr-form"],
    # GEMM accumulators in VGPRs; the indexer-query chain is explicit fmas
    "proj.hip": DEVICE + ["-ffp-contract=off"],
    "scratch.hip": DEVICE,
    "abi.cpp": ["-ffp-contract=off"],
}


def _compile(name, extra):
    src = os.path.join(CSRC, name)
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (name, " ".join(cmd), err))
    return obj, err


def build(verbose=False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        res = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    if verbose:
        for obj, err in res:
            if err.strip():
                print(err)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, *[o for o, _ in res], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stdout + r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
