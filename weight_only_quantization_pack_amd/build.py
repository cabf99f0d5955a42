"""Build libawq.so in-tree with hipcc for gfx950.

    python -m weight_only_quantization_pack_amd.build [--asm]

Every .hip source under csrc/ is compiled to an object in _build/ (in
parallel), then linked into weight_only_quantization_pack_amd/lib/libawq.so.
The measuring kernels under probe/ (a plain streaming read, the benchmark's
bandwidth reference; not part of the library) go into lib/libawq_probe.so.
--asm also keeps the gfx950 assembly of each source in _build/asm/.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(HERE, "lib")
ARCH = os.environ.get("AWQ_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # the quantizer's fp32 sequence must not be fused; FMAs are written explicitly
    "-ffp-contract=off",
    # no packed-fp32 VALU instructions anywhere in the library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the gfx feature flag: drop that warning only
    out = "\n".join(line for line in p.stdout.splitlines()
                    if "packed-fp32-ops" not in line and "is not a recognized feature" not in line)
    return p.returncode, out


def compile_one(src: str, asm: bool):
    name = os.path.splitext(os.path.basename(src))[0]
    obj = os.path.join(BUILD, name + ".o")
    rc, out = _run([HIPCC, *COMMON_FLAGS, "-c", src, "-o", obj])
    if rc != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if asm:
        adir = os.path.join(BUILD, "asm")
        os.makedirs(adir, exist_ok=True)
        rc, out2 = _run([HIPCC, *COMMON_FLAGS, "--cuda-device-only", "-S", src,
                         "-o", os.path.join(adir, name + ".s")])
        if rc != 0:
            raise RuntimeError(f"hipcc -S failed on {src}:\n{out2}")
    return obj, out


def build(asm: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    objs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for obj, out in ex.map(lambda s: compile_one(s, asm), srcs):
            objs.append(obj)
            if verbose and out.strip():
                print(out)
    lib = _link(objs, "libawq.so")
    probe_srcs = sorted(glob.glob(os.path.join(HERE, "probe", "*.hip")))
    if probe_srcs:
        _link([compile_one(s, asm)[0] for s in probe_srcs], "libawq_probe.so")
    return lib


def _link(objs, name):
    lib = os.path.join(LIBDIR, name)
    tmp = lib + ".tmp"
    rc, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError(f"link of {name} failed:\n{out}")
    os.replace(tmp, lib)
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(asm=a.asm, verbose=a.verbose))


if __name__ == "__main__":
    sys.exit(main())
