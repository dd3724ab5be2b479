"""Builds libcsa2.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m sparse_attention_fp4_kv_amd.build_lib
"""

import os
import shutil
import subprocess
import sys
import tempfile

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


# Per-source device flags.  The indexer's MFMA results feed VALU epilogues
# (ReLU and head weights), so its MFMAs are made to write VGPRs, never AGPRs
# (no v_accvgpr_read per result).  Elsewhere the compiler picks the form: the
# attention and CED accumulators land in VGPRs too (gfx950's register file is
# unified), the finish kernel's key-projection accumulators in AGPRs.
FILE_FLAGS = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    return err


def build(verbose=False):
    """Compile every HIP source into libcsa2.so next to this file (always rebuilds): one object
    per source (compiled in parallel, with its own flags), then one link."""
    tmp = LIB + ".tmp"
    objdir = tempfile.mkdtemp(prefix="csa2_build_")
    try:
        compile_flags = [f for f in FLAGS if f != "-shared"]
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(objdir, src + ".o")
            objs.append(obj)
            cmd = [hipcc()] + compile_flags + FILE_FLAGS.get(src, []) + ["-c", "-o", obj, os.path.join(CSRC, src)]
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        noise = "is not a recognized feature for this target"
        errs = []
        for cmd, p in procs:
            out, err = p.communicate()
            err = "\n".join(l for l in (err or "").splitlines() if noise not in l)
            if p.returncode != 0:
                raise RuntimeError("hipcc failed:\n" + err)
            errs.append(err)
        errs.append(_run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + LIBS))
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    err = "\n".join(e for e in errs if e.strip())
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
