"""Builds libcsa2.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m sparse_attention_fp4_kv_amd.build_lib
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsa2.so")
SOURCES = ["api.hip", "pack.hip", "indexer.hip", "attention.hip", "ced.hip", "latent.hip", "swa.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep hipcc from emitting packed-fp32 VALU ops (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# roctx (range markers around the C ABI calls, off unless CSA2_ROCTX is set)
LIBS = ["-lrocprofiler-sdk-roctx"]


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libcsa2 needs the ROCm toolchain to build")


def build(verbose=False):
    """Compile every HIP source into libcsa2.so next to this file (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + FLAGS + ["-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES] + LIBS
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
