"""The host-side code of libcsa2 (argument validation, workspace sizing, the launch timer, the block pool)
built with AddressSanitizer on the host pass only and exercised by tests/asan/abi_host_check.cpp on the
CPU (no call reaches a GPU).  ASan aborts the run on an out-of-bounds access, a use after free or a leak."""

import os
import shutil
import subprocess
import tempfile

import pytest

from sparse_attention_fp4_kv_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_under_asan():
    hipcc = build_lib.hipcc()
    tmp = tempfile.mkdtemp(prefix="csa2_asan_")
    try:
        exe = os.path.join(tmp, "abi_host_check")
        srcs = [os.path.join(build_lib.CSRC, s) for s in build_lib.SOURCES]
        cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
               "-o", exe, os.path.join(ROOT, "tests", "asan", "abi_host_check.cpp")] + srcs + build_lib.LIBS
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        assert res.returncode == 0, "\n".join(l for l in res.stderr.splitlines() if noise not in l)[-4000:]
        supp = os.path.join(tmp, "lsan.supp")
        with open(supp, "w") as f:  # leaks inside the ROCm runtime libraries are not this library's
            f.write("leak:libamdhip64\nleak:libhsa-runtime64\nleak:libhsakmt\nleak:librocprofiler\n")
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
                   LSAN_OPTIONS=f"suppressions={supp}")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
        assert "abi host checks ok" in run.stdout
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
