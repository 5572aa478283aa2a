"""Build libcassandra.so in-tree with hipcc for gfx950.

    python -m bit_level_weight_amd.build

Every .hip / .cpp file under csrc/ is compiled with the same flags and
linked into bit_level_weight_amd/libcassandra.so.  Device assembly of every
kernel file is also produced and screened (isa_check) before the library is
published, so that a kernel that writes through the scalar cache never ships.
"""
from __future__ import annotations

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
LIB = os.path.join(HERE, "libcassandra.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("command failed:\n  " + " ".join(cmd) + "\n" + p.stdout)
    return p.stdout


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *COMMON, "-x", "hip", "-c", src, "-o", obj]
    _run(cmd)
    asm = None
    if src.endswith(".hip"):
        asm = os.path.join(BUILD, os.path.basename(src) + ".s")
        _run([HIPCC, *COMMON, "--cuda-device-only", "-S", src, "-o", asm])
    return obj, asm


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    objs = [o for o, _ in results]
    asms = [a for _, a in results if a]
    from . import isa_check  # build-time screen, not needed at run time
    isa_check.check(asms)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "clean":
        shutil.rmtree(BUILD, ignore_errors=True)
    build()
