"""The quantizer decides a group's fp16 scale, its zero point and its codes
without divisions except near rounding boundaries (the device helpers in the
library's internal header).  tests/host/group_params_fastpath.c emulates those
decisions on the host (the reciprocal of D perturbed by one ulp either way, the
bound of v_rcp_f32) on random inputs and on inputs crafted within a few ulps of
the boundaries, and compares each with the IEEE division it replaces.  The GPU
side of the same cases is tests/test_gpu_quantize.py's boundary test."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = shutil.which("clang") or "/opt/rocm/lib/llvm/bin/clang"


def test_fast_paths_match_the_divisions(tmp_path):
    if not os.path.exists(CLANG):
        pytest.skip("no clang with _Float16 on the host")
    exe = str(tmp_path / "fastpath")
    subprocess.run([CLANG, "-O2", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "host", "group_params_fastpath.c"), "-lm"], check=True)
    r = subprocess.run([exe, "3000000"], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert " 0 differ" in r.stdout
