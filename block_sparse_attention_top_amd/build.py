"""Build libmsa.so (the HIP library behind include/msa.h) for gfx950 with hipcc.

Usage: python -m block_sparse_attention_top_amd.build   (or build() from Python)
The library is written next to this file; nothing is installed elsewhere.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["msa_api.hip", "msa_qcentric.hip", "msa_kvcentric.hip", "msa_combine.hip",
           "msa_csr.hip", "msa_decode.hip", "msa_decode_dense.hip",
           "msa_tile.hip", "msa_varlen.hip", "msa_decode_plan.hip"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 VALU forms are kept out of the generated code on purpose
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # no kernel computes on NaN (masked or out-of-range keys are zeroed or replaced
         # before any arithmetic), so fmaxf needs no NaN-quieting of its MFMA inputs;
         # infinities are still honoured (masking uses -inf)
         "-fno-honor-nans",
         "-Wall", "-Wno-unused-function"]


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed for {src}")
    noise = "is not a recognized feature for this target"
    for line in (res.stdout + res.stderr).splitlines():
        if noise not in line and line.strip():
            sys.stderr.write(line + "\n")


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libmsa.so; always rebuilds."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        list(ex.map(lambda a: _compile(*a), zip(SOURCES, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
