"""Build libcassandra.so in-tree with hipcc for gfx950.

    python -m bit_level_weight_amd.build          # release library
    python -m bit_level_weight_amd.build debug    # libcassandra_debug.so
    python -m bit_level_weight_amd.build all      # both

Every .hip / .cpp file under csrc/ is compiled with the same flags and
linked into bit_level_weight_amd/libcassandra.so.  Device assembly of every
kernel file is also produced and screened (isa_check) before the library is
published, so that a kernel that writes through the scalar cache never ships.
The debug library is the same sources compiled with CASS_DEBUG: device
bounds checks that record a flag instead of reading or writing out of range
(cass_debug_flags).
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
LIB_DEBUG = os.path.join(HERE, "libcassandra_debug.so")
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


def _compile(src, debug=False):
    out = os.path.join(BUILD, "debug") if debug else BUILD
    flags = COMMON + (["-DCASS_DEBUG"] if debug else [])
    obj = os.path.join(out, os.path.basename(src) + ".o")
    cmd = [HIPCC, *flags, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *flags, "-x", "hip", "-c", src, "-o", obj]
    _run(cmd)
    asm = None
    if src.endswith(".hip"):
        asm = os.path.join(out, os.path.basename(src) + ".s")
        _run([HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", asm])
    return obj, asm


def _sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _link(results, debug, verbose, nsrc):
    objs = [o for o, _ in results]
    asms = [a for _, a in results if a]
    from . import isa_check  # build-time screen, not needed at run time
    isa_check.check(asms)
    lib = LIB_DEBUG if debug else LIB
    tmp = lib + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {nsrc} sources")
    return lib


def build(verbose: bool = True, debug: bool = False) -> str:
    """One library: the release build, or with debug=True the CASS_DEBUG one."""
    os.makedirs(os.path.join(BUILD, "debug") if debug else BUILD, exist_ok=True)
    srcs = _sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, debug), srcs))
    return _link(results, debug, verbose, len(srcs))


def build_all(verbose: bool = True):
    """Both libraries, every compilation in one pool (the slowest files of the
    two builds overlap)."""
    os.makedirs(os.path.join(BUILD, "debug"), exist_ok=True)
    srcs = _sources()
    jobs = [(s, d) for d in (True, False) for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        results = list(ex.map(lambda j: _compile(*j), jobs))
    n = len(srcs)
    return (_link(results[n:], False, verbose, n), _link(results[:n], True, verbose, n))


if __name__ == "__main__":
    arg = sys.argv[1] if len(sys.argv) > 1 else ""
    if arg == "clean":
        shutil.rmtree(BUILD, ignore_errors=True)
    if arg == "all":
        build_all()
    else:
        build(debug=arg == "debug")
